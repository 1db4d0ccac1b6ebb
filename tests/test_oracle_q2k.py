"""Pins of the oracle's Q2_K routed experts.

The pages name Q2_K as the drafter's expert type (TensorSharp "Getting a
drafter", --expert-type q2_k) without defining it; the oracle reads GGUF's
Q2_K super-block as the format's public definition states it in words:
256 values in 84 bytes; bytes 0..15 = one byte per 16-value sub-block, scale
in the low nibble and min in the high nibble; bytes 16..79 = 2-bit quants, the
block's two 128-value halves 32 bytes each, value 32j + i of a half in bits
2j..2j+1 of the half's byte i; bytes 80..83 = fp16 d then fp16 dmin; a value
is d * scale * q - dmin * min.  The byte-level reading itself is not pinned by
any file of the pages (parity unpinned against a GGUF implementation); what
is pinned here is that the oracle decodes every position, scale and factor as
that description says, and that the layer uses the decoded matrices like a
dense numpy formulation does.
"""
import numpy as np
import pytest

import oracle
from mxfp4_routed_expert_sqrt_amd import synth
from mxfp4_routed_expert_sqrt_amd.configs import MoEShape
from tests.inputs import workload

Q2K_TINY = MoEShape("tiny_q2k", 32, 256, 16, 2, 256, "topk", "tiny_q2k")


def _block(qs=0, scales=0, d=0x3C00, dmin=0):
    b = np.zeros(84, dtype=np.uint8)
    b[16:80] = qs
    b[0:16] = scales
    b[80:82] = np.frombuffer(np.uint16(d).tobytes(), dtype=np.uint8)
    b[82:84] = np.frombuffer(np.uint16(dmin).tobytes(), dtype=np.uint8)
    return b


def test_half_decode_matches_numpy_float16():
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.half(int(b)) for b in bits[::5]])
    r = ref[::5]
    fin = np.isfinite(r)
    assert np.array_equal(got[fin], r[fin])
    assert np.array_equal(np.isnan(got), np.isnan(r))
    assert np.array_equal(np.isinf(got), np.isinf(r))


def test_uniform_blocks_closed_form():
    # block 0: q = 3 (0xFF), scale 1 / min 2 (0x21), d 0.5, dmin 0.25 -> 0.5*1*3 - 0.25*2 = 1
    # block 1: q = 1 (0x55), scale 3 / min 15 (0xF3), d 0.125, dmin 1/64 -> 0.375 - 0.234375
    row = np.concatenate([_block(0xFF, 0x21, 0x3800, 0x3400), _block(0x55, 0xF3, 0x3000, 0x2400)])
    w = oracle.decode_q2k(row[None, :], 512)[0]
    assert np.all(w[:256] == 1.0)
    assert np.all(w[256:] == 0.140625)


def test_every_quant_position():
    # one 2-bit field set to q = 2 at a time (scale 1, d 1): the value at the position the
    # format's description gives (byte 16 + 32*half + i, bits 2j) is 2, every other is 0
    seen = np.zeros(256, dtype=int)
    for half in range(2):
        for j in range(4):
            for i in range(32):
                b = _block(0, 0x01)
                b[16 + 32 * half + i] = 2 << (2 * j)
                w = oracle.decode_q2k(b[None, :], 256)[0]
                t = 128 * half + 32 * j + i
                assert w[t] == 2.0 and np.count_nonzero(w) == 1, (half, j, i)
                seen[t] += 1
    assert np.all(seen == 1)


def test_scale_and_min_of_each_sub_block():
    # sub-block m (values 16m..16m+15) takes byte m: scale m, min 15 - m; q = 3 everywhere
    sc = np.array([m | ((15 - m) << 4) for m in range(16)], dtype=np.uint8)
    b = _block(0xFF, sc, 0x3800, 0x3C00)  # d 0.5, dmin 1
    w = oracle.decode_q2k(b[None, :], 256)[0]
    m = np.arange(256) // 16
    assert np.array_equal(w, 0.5 * m * 3 - 1.0 * (15 - m))


def test_generator_quantiser_roundtrip():
    # the input generator's Q2_K quantiser decoded by the oracle: at most 4 levels per sub-block
    # (q in 0..3) and a 2-bit-sized error on Gaussian rows
    rng = np.random.default_rng(5)
    v = rng.standard_normal((8, 512)).astype(np.float32)
    w = oracle.decode_q2k(synth.encode_q2k(v), 512)
    assert max(len(np.unique(s)) for s in w.reshape(-1, 16)) <= 4
    rel = np.sqrt(np.mean((w - v) ** 2) / np.mean(v.astype(np.float64) ** 2))
    assert 0.1 < rel < 0.45
    # a row of equal non-negative values is exact: min 0, q = 3, d*scale = the value
    c = np.full((1, 256), 0.75, dtype=np.float32)
    assert np.allclose(oracle.decode_q2k(synth.encode_q2k(c), 256), 0.75, rtol=2e-3)


def _numpy_q2k_decode(blocks, K):
    """Vectorised decode of [R][K/256*84] from the format description (numpy float16 for the factors)."""
    R = blocks.shape[0]
    b = blocks.reshape(R, K // 256, 84)
    d = b[:, :, 80:82].copy().view(np.float16)[..., 0].astype(np.float64)
    dmin = b[:, :, 82:84].copy().view(np.float16)[..., 0].astype(np.float64)
    scale = (b[:, :, :16] & 15).astype(np.float64)
    mins = (b[:, :, :16] >> 4).astype(np.float64)
    qs = b[:, :, 16:80].reshape(R, K // 256, 2, 32)                     # [half][i]
    shifts = np.array([0, 2, 4, 6], dtype=np.uint8)
    q = (qs[:, :, :, None, :] >> shifts[None, None, None, :, None]) & 3  # [half][j][i]
    q = q.reshape(R, K // 256, 256).astype(np.float64)                  # t = 128 half + 32 j + i
    sub = np.arange(256) // 16
    return (d[..., None] * scale[:, :, sub] * q - dmin[..., None] * mins[:, :, sub]).reshape(R, K)


def test_numpy_decode_agrees_on_generated_experts():
    ex = synth.gen_experts_q2k(Q2K_TINY)
    for name, K in (("gate", 256), ("up", 256), ("down", 256)):
        m = ex[name][3]
        assert np.array_equal(oracle.decode_q2k(m, K), _numpy_q2k_decode(m, K))


@pytest.mark.parametrize("shared", ["bf16", "none"])
def test_q2k_layer_matches_dense_numpy(shared):
    sh = Q2K_TINY
    wl = workload(sh)
    ex = synth.gen_experts_q2k(sh)
    b = synth.gen_shared_bf16(sh) if shared == "bf16" else None
    r = oracle.forward(sh, wl["x"], wl["router_w"], wl["experts"], experts_q2k=ex, shared_bf16=b,
                       with_shared=shared == "bf16")
    f = lambda bits: (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    x = f(wl["x"])
    z = x @ wl["router_w"].astype(np.float64).T
    s = np.sqrt(np.logaddexp(0.0, z))
    top = np.sort(np.argsort(-s, axis=1, kind="stable")[:, :sh.top_k], axis=1)
    sel = np.take_along_axis(s, top, 1)
    mask = np.zeros((sh.n_rows, sh.n_experts))
    np.put_along_axis(mask, top, sel / sel.sum(1, keepdims=True), 1)
    L = sh.swiglu_limit

    def ffn(Wg, Wu, Wd):
        a, c = np.minimum(x @ Wg.T, L), np.clip(x @ Wu.T, -L, L)
        return (a / (1 + np.exp(-a)) * c) @ Wd.T

    ref = np.zeros((sh.n_rows, sh.d_model))
    for e in range(sh.n_experts):
        dec = {n: _numpy_q2k_decode(ex[n][e], sh.d_model if n != "down" else sh.d_ff) for n in ("gate", "up", "down")}
        ref += mask[:, e:e + 1] * ffn(dec["gate"], dec["up"], dec["down"])
    if b is not None:
        ref += ffn(f(b["gate"]), f(b["up"]), f(b["down"]))
    assert np.array_equal(r["idx"], top)
    assert np.allclose(r["out"], ref, rtol=1e-11, atol=1e-12 * np.abs(ref).max())
    assert np.abs(ref).max() > 0.05  # the routed experts contribute


def test_q2k_experts_equal_to_mxfp4_values_change_no_bit():
    # Q2_K blocks that hold exactly the values of MXFP4 rows give the MXFP4 layer's output: take a
    # Q2_K set, decode it, and re-encode those rows where MXFP4 represents them exactly (uniform fill)
    sh = Q2K_TINY
    wl = workload(sh)
    E, d, I = sh.n_experts, sh.d_model, sh.d_ff
    # every weight 1.0: MXFP4 code 2 with scale 127; Q2_K q 3, scale 1, min 2, d 0.5, dmin 0.25
    blk = _block(0xFF, 0x21, 0x3800, 0x3400)
    q2 = {"gate": np.tile(blk, (E, I, d // 256)), "up": np.tile(blk, (E, I, d // 256)),
          "down": np.tile(blk, (E, d, I // 256))}
    mx = dict(wl["experts"])
    for n, rows, K in (("gate", I, d), ("up", I, d), ("down", d, I)):
        mx[n + "_q"] = np.full((E + 1, rows, K // 2), 0x22, dtype=np.uint8)
        mx[n + "_s"] = np.full((E + 1, rows, K // 32), 127, dtype=np.uint8)
    r_mx = oracle.forward(sh, wl["x"], wl["router_w"], mx, with_shared=False)
    r_q2 = oracle.forward(sh, wl["x"], wl["router_w"], mx, experts_q2k=q2, with_shared=False)
    assert np.array_equal(r_mx["out"], r_q2["out"])
    assert np.abs(r_mx["out"]).max() > 0
