"""In-bounds checks of the gfx950 instruction behaviour the kernels assume.

- v_mfma_scale_f32_16x16x128_f8f6f4 (A = rows, B = columns, 128 K per step):
  * a 4-bit (E2M1) operand: lane l holds row/column l%16, K values
    32*(l/16) .. +31 as nibbles, low nibble first;
  * an 8-bit (E4M3) operand: lane l holds row/column l%16, K values
    16*(l/16) .. +15 in bytes 0..15 and 64 + 16*(l/16) .. +15 in bytes 16..31;
  * a 6-bit (E2M3) operand: lane l holds row/column l%16, K values
    32*(l/16) .. +31, value i in bits 6i .. 6i+5 of the little-endian bit
    string of dwords 0..5 (dwords 6 and 7 unused);
  * the E8M0 scale of row/column n and 32-block b (K 32b .. 32b+31) is the
    selected byte of the scale register of lane n + 16*b, for either format;
  * the fp32 result has D[4*(l/16)+i][l%16] in element i of lane l;
  * the instruction's internal sum is not fp32-exact: on 1024 random trials
    its error stayed below 2^-11 of the largest single product of the output
    (the bound checked here is 2^-10), which a wrong layout exceeds by far.
- v_cvt_pk_fp8_f32 rounds to the nearest E4M3 value (ties to even).
- The two-term FP6 split of a 32-value block (v_cvt_scalef32_2xpk16_fp6_f32
  and its unpack, as the prologue and the tall gate/up epilogue use them):
  codes are the nearest E2M3 values of v / 2^e (ties to the even code),
  value j at bits 6j of the operand, term 2 rounds the exact fp32 residual of
  term 1, and the exponents put each block maximum in (3.75, 7.5].
- permlane32/permlane16 swaps exchange the documented lane rows.
- moe_pack_mxfp4 and moe_pack_bf16 produce the packed layouts described in
  the C header.
- The streaming-read probe that the benchmark times (libmoe_hbm.so) reads
  every 16-byte piece of its buffer exactly once, whatever the grid.
Expected values come from independent numpy decoders written here.
"""
import ctypes
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

PROBE = os.path.join(os.path.dirname(__file__), "hip", "libmfma_probe.so")


def _lib():
    if not os.path.exists(PROBE):
        pytest.fail(f"{PROBE} not built (run __graft_entry__.build())")
    L = ctypes.CDLL(PROBE)
    L.probe_mfma.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int]
    L.probe_fp8.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int]
    L.probe_fp6.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int]
    L.probe_swap.argtypes = [ctypes.c_void_p] * 2
    return L


def e2m1(codes):
    codes = codes.astype(np.int64)
    sign = np.where(codes & 8, -1.0, 1.0)
    E, M = (codes >> 1) & 3, codes & 1
    return sign * np.where(E == 0, 0.5 * M, np.ldexp(1.0 + 0.5 * M, E - 1))


def e4m3(b):
    b = b.astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    E, M = (b >> 3) & 15, b & 7
    v = np.where(E == 0, np.ldexp(M / 8.0, -6), np.ldexp(1.0 + M / 8.0, E - 7))
    return np.where((E == 15) & (M == 7), np.nan, sign * v)


def e4m3_round(x):
    """Nearest E4M3 byte of each float (ties to the even code); |x| < 464."""
    grid_b = np.arange(0, 127, dtype=np.int64)  # non-negative finite codes 0x00..0x7E
    grid_v = e4m3(grid_b)
    out = np.empty(x.shape, dtype=np.int64)
    for n, v in enumerate(x.ravel()):
        a = abs(float(v))
        dist = np.abs(grid_v - a)
        best = np.flatnonzero(dist == dist.min())
        code = int(best[0]) if best.size == 1 else int(best[(grid_b[best] & 1) == 0][0])
        if np.signbit(v):
            code |= 0x80
        out.flat[n] = code
    return out


def _dense_fp4(a_bytes, scales):
    """[64 lanes][32 bytes] E2M1 operand -> dense [16][128] with per-(row, block) scales applied."""
    lo, hi = a_bytes[:, :16] & 15, a_bytes[:, :16] >> 4
    vals = e2m1(np.stack([lo, hi], -1).reshape(64, 32))
    M = np.zeros((16, 128))
    for l in range(64):
        M[l % 16, 32 * (l // 16):32 * (l // 16) + 32] = vals[l]
    return M * _block_scales(scales)


def _dense_fp8(b_bytes, scales):
    vals = e4m3(b_bytes)
    M = np.zeros((16, 128))
    for l in range(64):
        g = l // 16
        M[l % 16, 16 * g:16 * g + 16] = vals[l, :16]
        M[l % 16, 64 + 16 * g:64 + 16 * g + 16] = vals[l, 16:]
    return M * _block_scales(scales)


def e2m3(codes):
    codes = codes.astype(np.int64)
    sign = np.where(codes & 0x20, -1.0, 1.0)
    E, M = (codes >> 3) & 3, codes & 7
    return sign * np.where(E == 0, M / 8.0, np.ldexp(1.0 + M / 8.0, E - 1))


def _dense_fp6(b_bytes, scales):
    M = np.zeros((16, 128))
    for l in range(64):
        bits = int.from_bytes(b_bytes[l, :24].tobytes(), "little")
        codes = np.array([(bits >> (6 * i)) & 63 for i in range(32)])
        M[l % 16, 32 * (l // 16):32 * (l // 16) + 32] = e2m3(codes)
    return M * _block_scales(scales)


def _block_scales(scales):
    """Scale of (row n, block b) comes from lane n + 16 b."""
    S = np.zeros((16, 128))
    for n in range(16):
        for b in range(4):
            S[n, 32 * b:32 * b + 32] = np.ldexp(1.0, int(scales[n + 16 * b]) - 127)
    return S


def _lane_layout(D):
    return np.array([[D[4 * (l // 16) + i, l % 16] for i in range(4)] for l in range(64)])


@pytest.mark.parametrize("variant", [0, 1, 2, 3])
def test_scaled_mfma_layout(variant):
    print(f"probe_mfma variant {variant}", flush=True)
    rng = np.random.default_rng(10 + variant)
    a = rng.integers(0, 256, (64, 32), dtype=np.uint8)
    b = rng.integers(0, 256, (64, 32), dtype=np.uint8)
    if variant in (0, 1):
        b[(b & 0x7F) == 0x7F] = 0x3C  # no NaN encodings
    sa_w = rng.integers(0, 2 ** 32, 64, dtype=np.uint64).astype(np.uint32)
    sb_w = rng.integers(0, 2 ** 32, 64, dtype=np.uint64).astype(np.uint32)
    ja, jb = (2, 1) if variant == 1 else (0, 0)
    sa = rng.integers(118, 136, 64)
    sb = rng.integers(118, 136, 64)
    sa_w = (sa_w & ~np.uint32(0xFF << (8 * ja))) | (sa.astype(np.uint32) << np.uint32(8 * ja))
    sb_w = (sb_w & ~np.uint32(0xFF << (8 * jb))) | (sb.astype(np.uint32) << np.uint32(8 * jb))
    A = _dense_fp4(a, sa)
    B = {2: _dense_fp4, 3: _dense_fp6}.get(variant, _dense_fp8)(b, sb)
    exp = _lane_layout(A @ B.T)
    max_prod = _lane_layout(np.abs(A[:, None, :] * B[None, :, :]).max(-1))
    dev = torch.device("cuda")
    ta, tb = torch.from_numpy(a).to(dev), torch.from_numpy(b).to(dev)
    tsa, tsb = torch.from_numpy(sa_w.view(np.int32)).to(dev), torch.from_numpy(sb_w.view(np.int32)).to(dev)
    d = torch.zeros((64, 4), dtype=torch.float32, device=dev)
    assert _lib().probe_mfma(ta.data_ptr(), tb.data_ptr(), tsa.data_ptr(), tsb.data_ptr(), d.data_ptr(), variant) == 0
    got = d.cpu().numpy().astype(np.float64)
    worst = (np.abs(got - exp) / max_prod).max()
    print(f"variant {variant}: max |err| / max|product| = 2^{np.log2(max(worst, 1e-300)):.2f}", flush=True)
    assert worst <= 2.0 ** -10


def test_fp8_conversion_rounds_to_nearest_even():
    print("probe_fp8", flush=True)
    rng = np.random.default_rng(3)
    grid = e4m3(np.arange(0, 127))
    mids = (grid[1:] + grid[:-1]) / 2  # exact ties
    vals = np.concatenate([rng.uniform(-300, 300, 2048), rng.uniform(-1, 1, 1024) * 2.0 ** -7, mids, -mids,
                           grid, -grid, [0.0, -0.0, 255.9, 240.0, 1e-9]]).astype(np.float32)
    vals = vals[: (vals.size // 4) * 4]
    dev = torch.device("cuda")
    tin = torch.from_numpy(vals).to(dev)
    packed = torch.zeros(vals.size // 4, dtype=torch.int32, device=dev)
    back = torch.zeros(vals.size, dtype=torch.float32, device=dev)
    assert _lib().probe_fp8(tin.data_ptr(), packed.data_ptr(), back.data_ptr(), vals.size // 4) == 0
    got = packed.cpu().numpy().view(np.uint32)
    got_bytes = np.stack([(got >> (8 * i)) & 0xFF for i in range(4)], -1).reshape(-1)
    exp = e4m3_round(vals.astype(np.float64))
    bad = np.flatnonzero(got_bytes != exp)
    assert bad.size == 0, f"{bad.size} mismatches, e.g. {vals[bad[:5]]} -> {got_bytes[bad[:5]]} vs {exp[bad[:5]]}"
    assert np.array_equal(back.cpu().numpy().astype(np.float64), e4m3(exp))


def test_pack_layout_matches_header():
    from mxfp4_routed_expert_sqrt_amd import capi
    from mxfp4_routed_expert_sqrt_amd.layer import pack_mxfp4
    print("moe_pack_mxfp4", flush=True)
    rng = np.random.default_rng(4)
    for n_mat, rows, K in [(2, 32, 256), (1, 16, 128), (3, 48, 640)]:
        q = rng.integers(0, 256, (n_mat, rows, K // 2), dtype=np.uint8)
        s = rng.integers(0, 256, (n_mat, rows, K // 32), dtype=np.uint8)
        dev = torch.device("cuda")
        qo, so = pack_mxfp4(torch.from_numpy(q).to(dev), torch.from_numpy(s).to(dev), rows, K)
        torch.cuda.synchronize()
        qo, so = qo.cpu().numpy(), so.cpu().numpy()
        nks, n_sg = K // 128, (K // 128 + 3) // 4
        qb, sb = capi.moe_packed_mxfp4_bytes(rows, K)
        for m in range(n_mat):
            for rt in range(rows // 16):
                for ks in range(nks):
                    for lane in range(64):
                        row, blk = 16 * rt + lane % 16, 4 * ks + lane // 16
                        off = m * qb + (rt * nks + ks) * 1024 + lane * 16
                        assert np.array_equal(qo[off:off + 16], q[m, row, blk * 16:blk * 16 + 16])
                for sg in range(n_sg):
                    for lane in range(64):
                        off = m * sb + (rt * n_sg + sg) * 256 + lane * 4
                        for j in range(4):
                            ks = 4 * sg + j
                            want = s[m, 16 * rt + lane % 16, 4 * ks + lane // 16] if ks < nks else 127
                            assert qo is not None and so[off + j] == want


def e2m3(codes):
    codes = codes.astype(np.int64)
    sign = np.where(codes & 32, -1.0, 1.0)
    E, M = (codes >> 3) & 3, codes & 7
    return sign * np.where(E == 0, M / 8.0, np.ldexp(1.0 + M / 8.0, E - 1))


def e2m3_nearest(x):
    """Nearest E2M3 code of each value (ties to the even code), saturating at 7.5."""
    grid = e2m3(np.arange(32))  # non-negative codes 0..31, increasing
    a = np.minimum(np.abs(x), 7.5)
    d = np.abs(a[:, None] - grid[None, :])
    best = d.min(1, keepdims=True)
    cand = np.where(d == best, np.arange(32)[None, :], 99)
    even = np.where(cand % 2 == 0, cand, 99).min(1)
    code = np.where(even < 99, even, cand.min(1))
    return np.where((x < 0) & (code != 0), code | 32, code)


def fp6_exponent(amax):
    """Shared exponent e with amax / 2^e in (3.75, 7.5], clamped to [-126, 127] (0 for an all-zero block)."""
    if amax <= 0:
        return 0
    _, ex = np.frexp(amax)
    e = int(ex) - 3
    if amax > np.ldexp(7.5, e):
        e += 1
    return min(max(e, -126), 127)


def test_fp6_split_conversions():
    print("probe_fp6", flush=True)
    rng = np.random.default_rng(6)
    grid = e2m3(np.arange(32))
    mids = (grid[1:] + grid[:-1]) / 2  # exact ties at scale 1
    blocks = [rng.standard_normal(32) * 2.0 ** rng.integers(-20, 20) for _ in range(200)]
    blocks += [np.concatenate([mids, [7.5]]) * sgn for sgn in (1, -1)]  # 31 ties + the maximum: scale 2^0
    blocks += [np.zeros(32), np.full(32, 3.0), np.linspace(-7.5, 7.5, 32) * 2.0 ** -5]
    one_big = rng.standard_normal(32) * 2.0 ** -16
    one_big[7] = 1.7265625
    blocks.append(one_big)
    x = np.stack(blocks).astype(np.float32)
    n = x.shape[0]
    dev = torch.device("cuda")
    tin = torch.from_numpy(x.reshape(-1)).to(dev)
    codes = torch.zeros(n * 12, dtype=torch.int32, device=dev)
    exps = torch.zeros(n * 2, dtype=torch.int32, device=dev)
    res = torch.zeros(n * 32, dtype=torch.float32, device=dev)
    assert _lib().probe_fp6(tin.data_ptr(), codes.data_ptr(), exps.data_ptr(), res.data_ptr(), n) == 0
    got_w = codes.cpu().numpy().view(np.uint32).reshape(n, 2, 6)
    got_e = exps.cpu().numpy().reshape(n, 2)
    got_r = res.cpu().numpy().reshape(n, 32)
    for b in range(n):
        v = x[b]
        e1 = fp6_exponent(float(np.abs(v).max()))
        c1 = e2m3_nearest(v.astype(np.float64) / 2.0 ** e1)
        r = (v - (e2m3(c1) * 2.0 ** e1).astype(np.float32)).astype(np.float32)  # fp32 subtraction, as the kernel
        e2 = fp6_exponent(float(np.abs(r).max()))
        c2 = e2m3_nearest(r.astype(np.float64) / 2.0 ** e2)
        assert (got_e[b, 0], got_e[b, 1]) == (e1, e2), (b, got_e[b], e1, e2)
        assert np.array_equal(got_r[b], r), b
        for t, c in enumerate((c1, c2)):
            bits = sum(int(w) << (32 * i) for i, w in enumerate(got_w[b, t]))
            fields = np.array([(bits >> (6 * j)) & 63 for j in range(32)])
            # values compared (a value that rounds to zero may carry either sign bit)
            assert np.array_equal(e2m3(fields), e2m3(c)), (b, t, fields, c)
    # the ties block: every midpoint went to the even code
    assert got_e[n - 6, 0] == 0


def test_permlane_swaps():
    print("probe_swap", flush=True)
    dev = torch.device("cuda")
    x = np.arange(64, dtype=np.float32) + 1000
    y = np.arange(64, dtype=np.float32) + 2000
    out = torch.zeros(256, dtype=torch.float32, device=dev)
    assert _lib().probe_swap(torch.from_numpy(np.concatenate([x, y])).to(dev).data_ptr(), out.data_ptr()) == 0
    o = out.cpu().numpy().reshape(4, 64)
    x32, y32 = x.copy(), y.copy()
    x32[32:], y32[:32] = y[:32], x[32:]
    x16, y16 = x.copy(), y.copy()
    for base in (0, 32):
        x16[base + 16:base + 32], y16[base:base + 16] = y[base:base + 16], x[base + 16:base + 32]
    assert np.array_equal(o[0], x32) and np.array_equal(o[1], y32)
    assert np.array_equal(o[2], x16) and np.array_equal(o[3], y16)


def test_bf16_pack_layout_matches_header():
    from mxfp4_routed_expert_sqrt_amd.layer import pack_bf16
    print("moe_pack_bf16", flush=True)
    rng = np.random.default_rng(7)
    dev = torch.device("cuda")
    for n_mat, rows, K in [(1, 16, 32), (2, 48, 96), (3, 32, 512)]:
        w = rng.integers(-32768, 32768, (n_mat, rows, K), dtype=np.int16)
        out = pack_bf16(torch.from_numpy(w).to(dev), rows, K).cpu().numpy()
        torch.cuda.synchronize()
        assert out.size == w.nbytes
        o16 = out.view(np.int16).reshape(n_mat, -1)
        nks = K // 32
        for m in range(n_mat):
            for rt in range(rows // 16):
                for ks in range(nks):
                    frag = o16[m, (rt * nks + ks) * 512:(rt * nks + ks + 1) * 512].reshape(64, 8)
                    for lane in range(64):
                        row, k0 = 16 * rt + lane % 16, 32 * ks + 8 * (lane // 16)
                        assert np.array_equal(frag[lane], w[m, row, k0:k0 + 8]), (m, rt, ks, lane)


@pytest.mark.parametrize("nbytes,workgroups", [(1 << 20, 8), ((1 << 22) + 48, 64), (4096 * 16 * 8 + 16, 4096)])
def test_hbm_read_probe_reads_every_piece_once(nbytes, workgroups):
    # The XOR of the per-wave folds equals the XOR of every dword of the buffer only if each
    # 16-byte piece is read exactly once (a missed or repeated piece of random data changes it).
    path = os.path.join(os.path.dirname(os.path.dirname(__file__)), "mxfp4_routed_expert_sqrt_amd", "libmoe_hbm.so")
    if not os.path.exists(path):
        pytest.fail(f"{path} not built (run __graft_entry__.build())")
    L = ctypes.CDLL(path)
    L.hbm_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
                                 ctypes.c_void_p]
    L.hbm_probe_sink_words.argtypes = [ctypes.c_int]
    dev = torch.device("cuda:0")
    words = np.random.default_rng(nbytes).integers(0, 2 ** 32, nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).to(dev)
    want = np.bitwise_xor.reduce(words)
    stream = torch.cuda.current_stream(dev).cuda_stream
    for nt in (0, 1):
        sink = torch.zeros(L.hbm_probe_sink_words(workgroups), dtype=torch.int32, device=dev)
        assert L.hbm_read_probe(buf.data_ptr(), nbytes, nt, sink.data_ptr(), workgroups, stream) == 0
        torch.cuda.synchronize()
        got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
        assert got == want, (nbytes, workgroups, nt)

