"""Pins of the fp64 oracle to facts that do not come from the oracle itself.

Each test names what fixes the expected value: the OCP MX format definition,
library routines (numpy), closed forms, brute force on tiny inputs, invariants
of the layer, and the byte counts the pages print (tests/golden/).
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from mxfp4_routed_expert_sqrt_amd import synth
from mxfp4_routed_expert_sqrt_amd.configs import SHAPES, MoEShape
from tests.inputs import workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------- formats

def test_e2m1_matches_ocp_value_set():
    # OCP MX v1.0, E2M1: values {0, 0.5, 1, 1.5, 2, 3, 4, 6} with a sign bit;
    # max normal 6.0, min normal 1.0, only subnormal 0.5.
    vals = [oracle.e2m1(c) for c in range(16)]
    assert sorted(vals[:8]) == vals[:8]  # codes 0..7 increase
    assert set(vals[:8]) == {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0}
    assert vals[8:] == [-v for v in vals[:8]]
    assert math.copysign(1.0, vals[8]) == -1.0  # code 8 is -0
    assert max(vals) == 6.0 and min(v for v in vals if v > 0) == 0.5


def test_e8m0_is_power_of_two():
    for e in range(255):
        assert oracle.e8m0(e) == 2.0 ** (e - 127)
    assert math.isnan(oracle.e8m0(255))


def test_bf16_decode_matches_numpy():
    bits = np.arange(0, 65536, 7, dtype=np.uint32)
    with np.errstate(invalid="ignore"):
        ref = (bits << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    got = np.array([oracle.bf16(int(b)) for b in bits])
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite], ref[finite])
    assert np.array_equal(np.isnan(got), np.isnan(ref))


def test_nibble_order_and_scale():
    # element 2i is the low nibble of byte i; one scale per 32 elements
    q = np.zeros((1, 32), dtype=np.uint8)  # K = 64
    q[0, 0] = 0x21        # elem0 = code 1 (0.5), elem1 = code 2 (1.0)
    q[0, 16] = 0xF7       # elem32 = code 7 (6.0), elem33 = code 15 (-6.0)
    s = np.array([[127 + 3, 127 - 2]], dtype=np.uint8)
    w = oracle.decode_mxfp4(q, s)[0]
    assert w[0] == 0.5 * 8 and w[1] == 1.0 * 8
    assert w[32] == 6.0 / 4 and w[33] == -6.0 / 4
    assert np.count_nonzero(w) == 4


def test_generator_encoding_roundtrips_through_decode():
    # values already on the MXFP4 grid come back exactly (independent encoder)
    rng = np.random.default_rng(1)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float64)
    v = grid[rng.integers(0, 8, (8, 64))] * rng.choice([-1, 1], (8, 64))
    v[:, 0] = 6.0  # pin each block's max so the shared exponent is 0 ... then scale it
    v[:, 32] = -6.0
    scale = 2.0 ** rng.integers(-20, 20, (8, 1))
    vv = (v * scale).astype(np.float32)
    q, s = synth.encode_mxfp4(vv)
    assert np.array_equal(oracle.decode_mxfp4(q, s), vv.astype(np.float64))


def test_decoded_weight_statistics_follow_recipe():
    sh = SHAPES["tiny"]
    ex = synth.gen_experts(sh)
    w = oracle.decode_mxfp4(ex["gate_q"][3], ex["gate_s"][3])
    assert abs(w.std() * math.sqrt(sh.d_model) - 1.0) < 0.05
    dn = oracle.decode_mxfp4(ex["down_q"][3], ex["down_s"][3])
    assert abs(dn.std() * math.sqrt(sh.d_ff) - 1.0) < 0.05


# ------------------------------------------------------------------ router

def test_softplus_identities_and_asymptotes():
    for z in np.linspace(-30, 30, 121):
        assert abs(oracle.softplus(z) - oracle.softplus(-z) - z) < 1e-13
    assert oracle.score(0.0) == pytest.approx(0.8325546111576977, abs=1e-16)  # sqrt(ln 2)
    assert oracle.softplus(-40.0) / math.exp(-40.0) == pytest.approx(1.0, abs=1e-15)
    assert oracle.softplus(40.0) == 40.0
    zs = np.linspace(-20, 20, 401)
    sp = np.array([oracle.softplus(z) for z in zs])
    assert np.all(np.diff(sp) > 0)
    assert np.allclose(sp, np.logaddexp(0.0, zs), rtol=1e-15, atol=0)  # numpy's log(e^0 + e^z)


def test_router_logits_match_numpy_matmul():
    wl = workload("tiny")
    x = (wl["x"].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ref = x @ wl["router_w"].astype(np.float64).T
    z = oracle.router_logits(wl["x"], wl["router_w"])
    assert np.allclose(z, ref, rtol=1e-12, atol=1e-14)
    b = np.linspace(-1, 1, wl["shape"].n_experts).astype(np.float32)
    zb = oracle.router_logits(wl["x"], wl["router_w"], b)
    assert np.allclose(zb - z, b.astype(np.float64)[None, :], atol=1e-12)


def test_topk_brute_force_and_argsort():
    rng = np.random.default_rng(5)
    for E, k in [(16, 2), (256, 6), (8, 8), (33, 1)]:
        for _ in range(20):
            s = rng.random(E)
            idx, gap = oracle.topk(s, k)
            brute = sorted(sorted(range(E), key=lambda e: -s[e])[:k])
            assert list(idx) == brute
            assert list(idx) == sorted(np.argsort(-s, kind="stable")[:k].tolist())
            chosen = s[idx]
            rest = np.delete(s, idx)
            assert chosen.min() >= (rest.max() if rest.size else -np.inf)
            assert len(set(idx.tolist())) == k
            if k < E:
                assert gap == pytest.approx(chosen.min() - rest.max(), abs=0)


def test_topk_tie_goes_to_lower_id():
    s = np.array([1.0, 3.0, 2.0, 3.0, 2.0, 2.0])
    idx, gap = oracle.topk(s, 3)
    assert list(idx) == [1, 2, 3] and gap == 0.0


def test_gates_are_normalised_selected_scores():
    wl = workload("tiny")
    sh = wl["shape"]
    z = oracle.router_logits(wl["x"], wl["router_w"])
    idx, gates, margin = oracle.route(z, sh.top_k)
    s = np.sqrt(np.logaddexp(0.0, z))
    assert np.allclose(gates.sum(1), 1.0, atol=1e-15)
    assert np.all(gates > 0)
    sel = np.take_along_axis(s, idx.astype(np.int64), 1)
    assert np.allclose(gates, sel / sel.sum(1, keepdims=True), rtol=1e-14)
    assert np.all(np.diff(idx, axis=1) > 0)  # ascending expert id


def test_hash_routing_takes_table_rows():
    sh = MoEShape("t", 6, 64, 8, 3, 32, "hash", "tiny", vocab=5)
    table = np.array([[7, 1, 4], [0, 2, 5], [3, 6, 1], [5, 4, 3], [2, 7, 0]], dtype=np.int32)
    tok = np.array([4, 0, 0, 2, 3, 1], dtype=np.int32)
    z = np.random.default_rng(0).standard_normal((6, 8))
    idx, gates, margin = oracle.route(z, 3, "hash", tok, table)
    for r in range(6):
        assert list(idx[r]) == sorted(table[tok[r]].tolist())
    s = np.sqrt(np.logaddexp(0.0, z))
    sel = np.take_along_axis(s, idx.astype(np.int64), 1)
    assert np.allclose(gates, sel / sel.sum(1, keepdims=True), rtol=1e-14)
    assert np.all(np.isinf(margin))
    bad = table.copy()
    bad[4, 1] = 2  # duplicate id
    with pytest.raises(ValueError):
        oracle.route(z, 3, "hash", tok, bad)


# -------------------------------------------------------------- bookkeeping

def test_bookkeeping_brute_force():
    rng = np.random.default_rng(2)
    for N, k, E in [(32, 2, 16), (100, 6, 256), (7, 3, 4), (1, 1, 1)]:
        idx = np.stack([np.sort(rng.choice(E, k, replace=False)) for _ in range(N)]).astype(np.int32)
        counts, offsets, perm, inv = oracle.bookkeeping(idx, E)
        # brute force: list pairs expert by expert, rows ascending
        order = [r * k + j for e in range(E) for r in range(N) for j in range(k) if idx[r, j] == e]
        assert perm.tolist() == order
        assert counts.tolist() == [int((idx == e).sum()) for e in range(E)]
        assert offsets.tolist() == [0] + np.cumsum(counts).tolist()
        assert sorted(perm.tolist()) == list(range(N * k))
        assert np.array_equal(inv[perm], np.arange(N * k))
        for e in range(E):
            seg = perm[offsets[e]:offsets[e + 1]]
            assert np.all(idx.ravel()[seg] == e)
            assert np.all(np.diff(seg // k) > 0)


# ---------------------------------------------------------------- the layer

def _numpy_decode(q, s):
    """Independent vectorised MXFP4 decode (closed form of E2M1, power-of-two scales)."""
    codes = np.stack([q & 15, q >> 4], axis=-1).reshape(*q.shape[:-1], q.shape[-1] * 2).astype(np.int64)
    sign = np.where(codes & 8, -1.0, 1.0)
    E = (codes >> 1) & 3
    M = codes & 1
    mag = np.where(E == 0, 0.5 * M, np.ldexp(1.0 + 0.5 * M, E - 1))
    scale = np.ldexp(1.0, s.astype(np.int64) - 127)
    return sign * mag * np.repeat(scale, 32, axis=-1)


def _numpy_layer(shape, x_bits, w, ex, bias=None, route_scale=1.0, limit=10.0):
    """Dense formulation: every expert on every row, masked by the routing."""
    x = (x_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    z = x @ w.astype(np.float64).T
    if bias is not None:
        z = z + bias.astype(np.float64)
    s = np.sqrt(np.logaddexp(0.0, z))
    E, k = shape.n_experts, shape.top_k
    top = np.sort(np.argsort(-s, axis=1, kind="stable")[:, :k], axis=1)
    sel = np.take_along_axis(s, top, 1)
    g = sel / sel.sum(1, keepdims=True)
    mask = np.zeros((shape.n_rows, E))
    np.put_along_axis(mask, top, g, 1)
    out = np.zeros((shape.n_rows, shape.d_model))
    for e in range(E + 1):
        Wg = _numpy_decode(ex["gate_q"][e], ex["gate_s"][e])
        Wu = _numpy_decode(ex["up_q"][e], ex["up_s"][e])
        Wd = _numpy_decode(ex["down_q"][e], ex["down_s"][e])
        a, b = x @ Wg.T, x @ Wu.T
        if limit > 0:
            a, b = np.minimum(a, limit), np.clip(b, -limit, limit)
        y = (a / (1 + np.exp(-a)) * b) @ Wd.T
        out += y if e == E else route_scale * mask[:, e:e + 1] * y
    return out, top, g


def test_layer_matches_dense_numpy_formulation():
    wl = workload("tiny")
    r = oracle.forward(wl["shape"], wl["x"], wl["router_w"], wl["experts"])
    ref, top, g = _numpy_layer(wl["shape"], wl["x"], wl["router_w"], wl["experts"])
    assert np.array_equal(r["idx"], top)
    assert np.allclose(r["gates"], g, rtol=1e-13)
    assert np.allclose(r["out"], ref, rtol=1e-11, atol=1e-12 * np.abs(ref).max())


def test_layer_matches_dense_numpy_with_bias_and_scale():
    wl = workload("tiny")
    sh = wl["shape"]
    bias = np.linspace(-0.5, 0.5, sh.n_experts).astype(np.float32)[::-1].copy()
    r = oracle.forward(sh, wl["x"], wl["router_w"], wl["experts"], router_bias=bias, route_scale=1.5)
    ref, top, _ = _numpy_layer(sh, wl["x"], wl["router_w"], wl["experts"], bias=bias, route_scale=1.5)
    assert np.array_equal(r["idx"], top)
    assert np.allclose(r["out"], ref, rtol=1e-11, atol=1e-12 * np.abs(ref).max())


def _numpy_byte_table():
    """Both E2M1 values of every byte (low nibble first), from the closed form in _numpy_decode."""
    b = np.repeat(np.arange(256, dtype=np.uint8)[:, None], 16, axis=1)  # one 32-value block per byte
    return _numpy_decode(b, np.full((256, 1), 127, dtype=np.uint8))[:, :2]


def _numpy_decode_fast(q, s, table):
    """_numpy_decode through a 256-entry byte table (the same closed form, fast enough for V4 matrices)."""
    R = q.shape[0]
    return table[q].reshape(R, -1) * np.repeat(np.ldexp(1.0, s.astype(np.int64) - 127), 32, axis=-1)


@pytest.mark.slow
def test_layer_matches_dense_numpy_at_v4_scale():
    # The oracle at the V4 layer's own sizes (d 4096, 256 experts top-6 + shared, I 2048; 512-row
    # verify batch): 16 rows spread over the batch, first and last included, against the dense numpy
    # fp64 formulation restricted to those rows (every expert they touch, masked by the routing),
    # and the whole batch's bookkeeping against numpy's stable argsort.  Sizes where index arithmetic
    # could overflow or an (expert, feature) work split could go wrong only show up here.
    wl = workload("verify512")
    sh, ex = wl["shape"], wl["experts"]
    E, k, d = sh.n_experts, sh.top_k, sh.d_model
    rows = np.unique(np.linspace(0, sh.n_rows - 1, 16).astype(np.int32))
    r = oracle.forward(sh, wl["x"], wl["router_w"], ex, rows=rows)

    x = (wl["x"][rows].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    s = np.sqrt(np.logaddexp(0.0, x @ wl["router_w"].astype(np.float64).T))
    top = np.sort(np.argsort(-s, axis=1, kind="stable")[:, :k], axis=1)
    sel = np.take_along_axis(s, top, 1)
    g = sel / sel.sum(1, keepdims=True)
    assert np.array_equal(r["idx"][rows], top)
    assert np.allclose(r["gates"][rows], g, rtol=1e-13)

    mask = np.zeros((len(rows), E))
    np.put_along_axis(mask, top, g, 1)
    table = _numpy_byte_table()
    out = np.zeros((len(rows), d))
    for e in sorted(set(top.ravel().tolist())) + [E]:
        Wg = _numpy_decode_fast(ex["gate_q"][e], ex["gate_s"][e], table)
        Wu = _numpy_decode_fast(ex["up_q"][e], ex["up_s"][e], table)
        Wd = _numpy_decode_fast(ex["down_q"][e], ex["down_s"][e], table)
        a = np.minimum(x @ Wg.T, sh.swiglu_limit)
        b = np.clip(x @ Wu.T, -sh.swiglu_limit, sh.swiglu_limit)
        y = (a / (1 + np.exp(-a)) * b) @ Wd.T
        out += y if e == E else mask[:, e:e + 1] * y
    assert np.allclose(r["out"], out, rtol=1e-11, atol=1e-12 * np.abs(out).max())

    idx = r["idx"].ravel()
    perm = np.argsort(idx, kind="stable")  # expert-major; pairs r*k+j ascending inside an expert
    counts = np.bincount(idx, minlength=E)
    _, off, p, inv = oracle.bookkeeping(r["idx"], E)
    assert np.array_equal(p, perm) and np.array_equal(off, np.concatenate([[0], np.cumsum(counts)]))
    assert np.array_equal(inv[perm], np.arange(sh.n_rows * k))
    assert np.array_equal(r["perm"], perm) and np.array_equal(r["counts"], counts)


def _single_entry_experts(sh, entries):
    """Weights that are zero except listed (matrix, expert, row, col) = 1.0 entries."""
    E, d, I = sh.n_experts, sh.d_model, sh.d_ff
    ex = {}
    for name, R, K in [("gate", I, d), ("up", I, d), ("down", d, I)]:
        ex[name + "_q"] = np.zeros((E + 1, R, K // 2), dtype=np.uint8)
        ex[name + "_s"] = np.full((E + 1, R, K // 32), 127, dtype=np.uint8)
    for name, e, row, col in entries:
        code = 2  # E2M1 code 2 is exactly 1.0; scale byte 127 is 2^0
        ex[name + "_q"][e, row, col // 2] |= code << (4 * (col % 2))
    return ex


def _bf16_bits(v):
    return (np.asarray(v, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_closed_form_single_weight_ffn():
    # one routed expert (k=1 of 2) and the shared expert, each with one 1.0 entry per matrix:
    # h_n = silu(x_i) * x_j and y_m = h_n, all other outputs exactly 0
    sh = MoEShape("t", 4, 64, 2, 1, 32, "topk", "tiny", swiglu_limit=0.0)
    ex = _single_entry_experts(sh, [("gate", 1, 5, 3), ("up", 1, 5, 10), ("down", 1, 7, 5),
                                    ("gate", 2, 0, 1), ("up", 2, 0, 2), ("down", 2, 60, 0)])
    x = np.zeros((4, 64), dtype=np.float32)
    x[:, 3] = [0.5, -1.25, 2.0, 3.0]
    x[:, 10] = [1.5, 2.0, -0.75, 0.25]
    x[:, 1] = [1.0, -2.0, 0.375, 4.0]
    x[:, 2] = [0.5, 0.5, -1.0, 2.0]
    w = np.zeros((2, 64), dtype=np.float32)
    w[1, 20] = 1.0
    x[:, 20] = 1.0  # expert 1 wins every row: logits (0, 1)
    r = oracle.forward(sh, _bf16_bits(x), w, ex)
    assert np.all(r["idx"][:, 0] == 1) and np.all(r["gates"] == 1.0)
    silu = lambda v: v / (1.0 + math.exp(-v))
    for row in range(4):
        exp = np.zeros(64)
        exp[7] = silu(float(x[row, 3])) * float(x[row, 10])
        exp[60] = silu(float(x[row, 1])) * float(x[row, 2])
        assert np.array_equal(r["out"][row], exp)


def test_swiglu_limit_clamps_gate_above_and_up_both_sides():
    sh = MoEShape("t", 2, 64, 2, 1, 32, "topk", "tiny", swiglu_limit=10.0)
    ex = _single_entry_experts(sh, [("gate", 1, 0, 3), ("up", 1, 0, 4), ("down", 1, 0, 0)])
    x = np.zeros((2, 64), dtype=np.float32)
    x[:, 3] = [12.0, -12.0]   # gate: 12 -> 10 ; -12 stays (no lower clamp)
    x[:, 4] = [-15.0, 16.0]   # up: -15 -> -10 ; 16 -> 10
    x[:, 20] = 1.0
    w = np.zeros((2, 64), dtype=np.float32)
    w[1, 20] = 1.0
    r = oracle.forward(sh, _bf16_bits(x), w, ex, with_shared=False)
    silu = lambda v: v / (1.0 + math.exp(-v))
    assert r["out"][0, 0] == silu(10.0) * -10.0
    assert r["out"][1, 0] == silu(-12.0) * 10.0
    r0 = oracle.forward(sh, _bf16_bits(x), w, ex, with_shared=False, swiglu_limit=0.0)
    assert r0["out"][0, 0] == silu(12.0) * -15.0


def test_identical_experts_reduce_to_scaled_shared():
    # if every routed expert equals the shared one, out = (1 + rs) * FFN(x) since sum g = 1
    wl = workload("tiny")
    sh = wl["shape"]
    ex = {k: np.repeat(v[-1:], sh.n_experts + 1, axis=0) for k, v in wl["experts"].items()}
    full = oracle.forward(sh, wl["x"], wl["router_w"], ex, route_scale=1.5)["out"]
    shared_only = oracle.forward(sh, wl["x"], wl["router_w"], ex, route_scale=0.0)["out"]
    assert np.allclose(full, 2.5 * shared_only, rtol=1e-13, atol=1e-15)


def test_zero_row_gives_zero_output_and_rows_are_independent():
    wl = workload("tiny")
    sh = wl["shape"]
    x = wl["x"].copy()
    x[5] = 0
    r = oracle.forward(sh, x, wl["router_w"], wl["experts"])
    assert np.all(r["out"][5] == 0.0)
    perm = np.random.default_rng(3).permutation(sh.n_rows)
    rp = oracle.forward(sh, x[perm].copy(), wl["router_w"], wl["experts"])
    assert np.array_equal(rp["out"], r["out"][perm])  # bit-exact row-permutation invariance
    assert np.array_equal(rp["idx"], r["idx"][perm])


def test_row_subset_and_thread_count_do_not_change_bits():
    wl = workload("tiny")
    sh = wl["shape"]
    a = oracle.forward(sh, wl["x"], wl["router_w"], wl["experts"], threads=1)
    b = oracle.forward(sh, wl["x"], wl["router_w"], wl["experts"], threads=7)
    rows = [31, 0, 17, 17, 4]
    c = oracle.forward(sh, wl["x"], wl["router_w"], wl["experts"], rows=rows, threads=3)
    assert np.array_equal(a["out"], b["out"])
    assert np.array_equal(c["out"], a["out"][rows])
    for key in ("idx", "perm", "offsets", "inv"):
        assert np.array_equal(a[key], c[key])


def test_constant_hash_table_routes_every_row_alike():
    sh = MoEShape("h", 32, 256, 16, 2, 128, "hash", "tiny", vocab=50)
    wl = workload("tiny")
    table = np.tile(np.array([[9, 3]], dtype=np.int32), (50, 1))
    tok = np.random.default_rng(4).integers(0, 50, 32).astype(np.int32)
    r = oracle.forward(sh, wl["x"], wl["router_w"], wl["experts"], token_ids=tok, tid2eid=table)
    assert np.all(r["idx"] == [3, 9])
    assert r["counts"][3] == 32 and r["counts"][9] == 32 and r["counts"].sum() == 64


def test_zipf_calibration_reaches_the_skew_targets():
    # the calibrated bias steers the per-row selection probability towards q_e = min(1, c * rank^-1.2),
    # sum q = 6: the hottest expert on (nearly) every row, i.e. (nearly) 1/6 of all assignments, the cap
    # that 6 distinct experts per row allow
    from tests.inputs import calibrate_zipf_bias
    sh = SHAPES["zipf2048"]
    x, w = synth.gen_x(sh), synth.gen_router(sh)
    b, q = calibrate_zipf_bias(sh, x, w)
    assert np.isclose(q.sum(), sh.top_k) and q.max() == 1.0
    idx, _, _ = oracle.route(oracle.router_logits(x, w, b), sh.top_k)
    q_hat = np.bincount(idx.ravel(), minlength=sh.n_experts) / sh.n_rows
    assert q_hat[np.argmax(q)] >= 0.95
    assert np.abs(q_hat - q).sum() < 0.2
    order = np.argsort(-q)  # the load falls with the target rank
    assert np.all(np.diff(q_hat[order[:8]]) <= 0.02)


def test_tiny_workload_margins():
    wl = workload("tiny")
    z = oracle.router_logits(wl["x"], wl["router_w"])
    _, _, margin = oracle.route(z, wl["shape"].top_k)
    assert margin.min() >= 1e-3


# -------------------------------------------------------------- byte model

def test_byte_model_matches_pages():
    with open(os.path.join(GOLDEN, "byte_model.json")) as f:
        g = json.load(f)
    sh = SHAPES["verify512"]
    d, I = sh.d_model, sh.d_ff
    per_matrix = d * I // 2 + d * I // 32  # nibbles + one E8M0 byte per 32
    per_expert = 3 * per_matrix
    assert per_expert == g["expert_payload_bytes"]["value"]
    assert abs(per_expert / 1e6 - g["expert_payload_mb_printed"]["value"]) < 0.05
    assert abs(sh.top_k * per_expert / 1e6 - g["routed_mb_per_token_printed"]["value"]) < 1.0
    total_gib = g["layers"]["value"] * sh.n_experts * per_expert / 2 ** 30
    assert abs(total_gib - g["routed_expert_gib_printed"]["value"]) < 0.5
    assert abs(sh.n_experts * 3 * d * I / 1e9 - g["params_per_layer_billion_printed"]["value"]) < 0.01


# ------------------------------------------------- input RMSNorm and residual

def _bf16_f32(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def test_rmsnorm_matches_torch_rms_norm():
    # A library routine of the same definition (fp32, its own reduction order): the bf16
    # results agree except where the two fp32 values straddle a bf16 rounding boundary.
    torch = pytest.importorskip("torch")
    sh = MoEShape("n", 64, 256, 16, 2, 128, "topk", "tiny")
    rng = np.random.default_rng(21)
    x = synth.scale_rows_bf16(synth.bf16_bits(rng.standard_normal((64, 256))), rng.integers(-3, 4, 64))
    g = synth.bf16_bits(1.0 + 0.1 * rng.standard_normal(256))
    ours = oracle.rmsnorm_bf16(x, g, 1e-6)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(_bf16_f32(x)), (256,), torch.from_numpy(_bf16_f32(g)),
                                       eps=1e-6)
    ref_bits = synth.bf16_bits(ref.numpy())
    diff = np.abs(ours.astype(np.int32) - ref_bits.astype(np.int32))
    assert diff.max() <= 1 and (diff > 0).mean() < 1e-2
    assert sh.d_model == 256


def test_rmsnorm_closed_forms():
    d = 128
    g1 = synth.bf16_bits(np.ones(d))
    # constant rows +-2^k with eps 0: x / sqrt(mean x^2) = +-1 exactly
    for c in (0.25, 1.0, -8.0):
        x = synth.bf16_bits(np.full((1, d), c))
        assert np.all(_bf16_f32(oracle.rmsnorm_bf16(x, g1, 0.0)) == np.sign(c))
    # power-of-two scaling of a row changes no bit (eps 0: every fp32 step scales exactly)
    rng = np.random.default_rng(5)
    x = synth.bf16_bits(rng.standard_normal((4, d)))
    g = synth.bf16_bits(1.0 + 0.1 * rng.standard_normal(d))
    a = oracle.rmsnorm_bf16(x, g, 0.0)
    b = oracle.rmsnorm_bf16(synth.scale_rows_bf16(x, np.array([5, -7, 1, 3])), g, 0.0)
    assert np.array_equal(a, b)
    # the weight multiplies elementwise: a weight of 2 doubles every element exactly
    g2 = synth.bf16_bits(np.full(d, 2.0))
    assert np.array_equal(_bf16_f32(oracle.rmsnorm_bf16(x, g2, 0.0)), 2 * _bf16_f32(oracle.rmsnorm_bf16(x, g1, 0.0)))
    # eps dominates a zero row: the output is exactly zero
    assert np.all(_bf16_f32(oracle.rmsnorm_bf16(np.zeros((1, d), np.uint16), g, 1e-6)) == 0)


def test_norm_forward_is_forward_on_normalised_rows_plus_residual():
    from tests.inputs import norm_workload
    wl = norm_workload("tiny")
    sh = wl["shape"]
    a = oracle.forward(sh, wl["x"], wl["router_w"], wl["experts"], norm_w=wl["norm_w"], norm_eps=wl["norm_eps"],
                       residual=wl["residual"])
    xn = oracle.rmsnorm_bf16(wl["x"], wl["norm_w"], wl["norm_eps"])
    b = oracle.forward(sh, xn, wl["router_w"], wl["experts"])
    for key in ("idx", "gates", "perm", "inv", "offsets"):
        assert np.array_equal(a[key], b[key])
    res = _bf16_f32(wl["residual"]).astype(np.float64)
    assert np.allclose(a["out"] - b["out"], res, rtol=0, atol=1e-12)
    # a zero norm weight zeroes the FFN input, so only the residual is left
    z = oracle.forward(sh, wl["x"], wl["router_w"], wl["experts"], norm_w=np.zeros(sh.d_model, np.uint16),
                       norm_eps=wl["norm_eps"], residual=wl["residual"])
    assert np.array_equal(z["out"], res)


def test_norm_workload_margins():
    from tests.inputs import norm_workload
    wl = norm_workload("tiny")
    xn = oracle.rmsnorm_bf16(wl["x"], wl["norm_w"], wl["norm_eps"])
    _, _, margin = oracle.route(oracle.router_logits(xn, wl["router_w"]), wl["shape"].top_k)
    assert margin.min() >= 1e-3
    assert len(set(synth.gen_row_exponents(wl["shape"]).tolist())) > 3


# --------------------------------------------------- selection-only router bias

def test_selection_only_bias_brute_force():
    # bias_mode 1: the k largest s + b choose the experts; the gates are the chosen unbiased
    # scores normalised (numpy: logits by matmul, s = sqrt(log(1 + e^z)), stable argsort)
    wl = workload("tiny")
    sh = wl["shape"]
    b = np.random.default_rng(8).normal(0, 0.05, sh.n_experts).astype(np.float32)
    r = oracle.forward(sh, wl["x"], wl["router_w"], wl["experts"], router_bias=b, bias_mode=1)
    x = _bf16_f32(wl["x"]).astype(np.float64)
    z = x @ wl["router_w"].astype(np.float64).T
    s = np.sqrt(np.logaddexp(0.0, z))
    t = s + b.astype(np.float64)[None, :]
    for row in range(sh.n_rows):
        want = np.sort(np.argsort(-t[row], kind="stable")[:sh.top_k])
        assert np.array_equal(r["idx"][row], want)
        g = s[row, want] / s[row, want].sum()
        assert np.allclose(r["gates"][row], g, rtol=1e-12, atol=0)
    assert np.allclose(r["z"], z, rtol=1e-12, atol=1e-12)  # the logits carry no bias in this mode


def test_selection_only_bias_zero_and_forcing():
    wl = workload("tiny")
    sh = wl["shape"]
    plain = oracle.forward(sh, wl["x"], wl["router_w"], wl["experts"])
    zero = oracle.forward(sh, wl["x"], wl["router_w"], wl["experts"], router_bias=np.zeros(sh.n_experts, np.float32),
                          bias_mode=1)
    for key in ("out", "idx", "gates", "perm"):
        assert np.array_equal(plain[key], zero[key])
    # a large bias on expert 5 puts it in every row; its gate stays its unbiased score's share
    b = np.zeros(sh.n_experts, np.float32)
    b[5] = 100.0
    forced = oracle.forward(sh, wl["x"], wl["router_w"], wl["experts"], router_bias=b, bias_mode=1)
    assert np.all((forced["idx"] == 5).any(axis=1))
    s = np.sqrt(np.logaddexp(0.0, forced["z"]))
    col = np.argmax(forced["idx"] == 5, axis=1)
    g5 = forced["gates"][np.arange(sh.n_rows), col]
    assert np.allclose(g5, s[:, 5] / np.take_along_axis(s, forced["idx"], 1).sum(1), rtol=1e-12)
    assert g5.max() < 0.9  # not dominated by the bias


# ------------------------------------------------------- bf16 shared expert

def _bf16_exact_bits(v):
    """fp64 values that bf16 holds exactly -> bit patterns (asserts the exactness)."""
    v = np.asarray(v, dtype=np.float64)
    f = v.astype(np.float32)
    assert np.array_equal(f.astype(np.float64), v)
    u = f.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0)
    return (u >> 16).astype(np.uint16)


def test_bf16_shared_expert_holding_the_mxfp4_values_changes_no_bit():
    # MXFP4 values have at most two significant bits and a power-of-two scale, so a bf16 copy of the
    # shared expert (decoded here independently of the oracle) holds them exactly: the layer is the same
    wl = workload("tiny")
    sh, ex = wl["shape"], wl["experts"]
    E = sh.n_experts
    b = {n: _bf16_exact_bits(_numpy_decode(ex[n + "_q"][E], ex[n + "_s"][E])) for n in ("gate", "up", "down")}
    r_mx = oracle.forward(sh, wl["x"], wl["router_w"], ex)
    r_bf = oracle.forward(sh, wl["x"], wl["router_w"], ex, shared_bf16=b)
    assert np.array_equal(r_mx["idx"], r_bf["idx"])
    assert np.array_equal(r_mx["out"], r_bf["out"])


@pytest.mark.parametrize("limit", [10.0, 0.05])
def test_bf16_shared_expert_matches_dense_numpy(limit):
    # the layer minus the layer without a shared expert is the shared FFN; here computed densely from
    # the bf16 weights (gate/up [I][d], down [d][I]); at limit 0.05 the clamp binds on most units
    wl = workload("tiny")
    sh = wl["shape"]
    b = synth.gen_shared_bf16(sh)
    r = oracle.forward(sh, wl["x"], wl["router_w"], wl["experts"], shared_bf16=b, swiglu_limit=limit)
    r0 = oracle.forward(sh, wl["x"], wl["router_w"], wl["experts"], with_shared=False, swiglu_limit=limit)
    f = lambda bits: (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    x = f(wl["x"])
    a, c = x @ f(b["gate"]).T, x @ f(b["up"]).T
    if limit == 0.05:
        assert np.mean(np.abs(a) > limit) > 0.5
    a, c = np.minimum(a, limit), np.clip(c, -limit, limit)
    y = (a / (1.0 + np.exp(-a)) * c) @ f(b["down"]).T
    assert np.array_equal(r["idx"], r0["idx"])
    assert np.allclose(r["out"] - r0["out"], y, rtol=1e-9, atol=1e-12 * np.abs(y).max())
