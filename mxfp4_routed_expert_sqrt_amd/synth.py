"""Seeded synthetic inputs for the routed MoE layer (Python side of csrc/synth.c).

Everything here is input generation: random draws and their encoding into the
formats the layer reads.  None of the layer's arithmetic lives here; where an
input recipe needs routing decisions (the top-k margin filter, the Zipf bias
calibration) the caller passes in the function that makes them.

Recipe (seed 0 unless stated):
- x: N(0, 1) per element, rounded to bf16; a row may be redrawn (attempt a+1)
  by a caller-supplied filter.
- router weight: N(0, 0.02) fp32 [E][d].
- experts 0..E-1 routed and expert E = the shared expert: gate/up N(0, 1/sqrt(d)),
  down N(0, 1/sqrt(I)), fp32 then MXFP4 (E2M1 + per-32 E8M0).
- hash routing: tid2eid [vocab][k] with k distinct ids per token id, token ids
  uniform over the vocabulary.
- Zipf load: per-row selection probability q_e = min(1, c * rank_e^-1.2) with
  sum q = k; ranks map to a seeded permutation of the experts.
- with the input RMSNorm: x rows scaled by 2^u, u uniform in {-3, ..., 3}
  (exact in bf16); norm weight 1 + N(0, 0.1) and residual N(0, 1), both bf16.
- selection-only router bias: N(0, 0.05) fp32 per expert.
"""
import ctypes
import os
import zlib

import numpy as np

from .configs import CFG_TAG, ROUTER_STD, SET_TAG, MoEShape, expert_std

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmoe_synth.so")
_lib = None

MAT_GATE, MAT_UP, MAT_DOWN = 1, 2, 3


def _cfg_tag(shape: MoEShape) -> int:
    return CFG_TAG[shape.name] if shape.name in CFG_TAG else 1000 + zlib.crc32(shape.name.encode())


def _set_tag(shape: MoEShape) -> int:
    return SET_TAG[shape.weight_set] if shape.weight_set in SET_TAG else 2000 + zlib.crc32(shape.weight_set.encode())


def usable_cpus() -> int:
    """CPUs this process may run on: affinity mask, capped by a cgroup v2 quota."""
    n = len(os.sched_getaffinity(0))
    try:
        with open("/sys/fs/cgroup/cpu.max") as f:
            quota, period = f.read().split()[:2]
        if quota != "max":
            n = max(1, min(n, int(int(quota) // int(period))))
    except (OSError, ValueError):
        pass
    return max(1, n)


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(_LIB_PATH)
        u64, i64, i32, dbl, vp = ctypes.c_uint64, ctypes.c_long, ctypes.c_int, ctypes.c_double, ctypes.c_void_p
        lib.synth_x_bf16.argtypes = [u64, u64, i64, i64, vp, vp, i32]
        lib.synth_router_f32.argtypes = [u64, u64, i64, i64, dbl, vp, i32]
        lib.synth_mxfp4.argtypes = [u64, u64, u64, i64, i64, i64, i64, dbl, vp, vp, i32]
        lib.synth_mxfp4.restype = i32
        lib.synth_q2k.argtypes = [u64, u64, u64, i64, i64, i64, i64, dbl, vp, i32]
        lib.synth_q2k.restype = i32
        lib.synth_encode_q2k.argtypes = [vp, i64, i64, vp]
        lib.synth_encode_mxfp4.argtypes = [vp, i64, i64, vp, vp]
        lib.synth_tid2eid.argtypes = [u64, u64, i64, i32, i32, vp, i32]
        lib.synth_tid2eid.restype = i32
        lib.synth_token_ids.argtypes = [u64, u64, i64, i64, vp]
        lib.synth_permutation.argtypes = [u64, u64, i64, vp]
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def gen_x(shape: MoEShape, seed: int = 0, attempts=None, threads=None) -> np.ndarray:
    """x [N][d] as bf16 bit patterns (uint16)."""
    out = np.empty((shape.n_rows, shape.d_model), dtype=np.uint16)
    att = None
    if attempts is not None:
        att = np.ascontiguousarray(attempts, dtype=np.int32)
        assert att.shape == (shape.n_rows,)
    _load().synth_x_bf16(seed, _cfg_tag(shape), shape.n_rows, shape.d_model,
                         _ptr(att) if att is not None else None, _ptr(out), threads or usable_cpus())
    return out


def gen_router(shape: MoEShape, seed: int = 0, threads=None) -> np.ndarray:
    out = np.empty((shape.n_experts, shape.d_model), dtype=np.float32)
    _load().synth_router_f32(seed, _set_tag(shape), shape.n_experts, shape.d_model,
                             ROUTER_STD, _ptr(out), threads or usable_cpus())
    return out


def gen_mxfp4(set_tag: int, mat_tag: int, first: int, count: int, rows: int, K: int, std: float,
              seed: int = 0, threads=None):
    q = np.empty((count, rows, K // 2), dtype=np.uint8)
    s = np.empty((count, rows, K // 32), dtype=np.uint8)
    rc = _load().synth_mxfp4(seed, set_tag, mat_tag, first, count, rows, K, std, _ptr(q), _ptr(s),
                             threads or usable_cpus())
    if rc != 0:
        raise ValueError("synth_mxfp4: bad shape")
    return q, s


_EXPERT_CACHE = {}


def gen_experts(shape: MoEShape, seed: int = 0, threads=None) -> dict:
    """Routed experts 0..E-1 and the shared expert (index E) in natural layout.

    Returns gate_q/up_q [E+1][I][d/2], gate_s/up_s [E+1][I][d/32],
    down_q [E+1][d][I/2], down_s [E+1][d][I/32] (uint8).  Cached per process.
    """
    key = (shape.weight_set, shape.n_experts, shape.d_model, shape.d_ff, seed)
    if key in _EXPERT_CACHE:
        return _EXPERT_CACHE[key]
    st = _set_tag(shape)
    E, d, I = shape.n_experts, shape.d_model, shape.d_ff
    w = {}
    w["gate_q"], w["gate_s"] = gen_mxfp4(st, MAT_GATE, 0, E + 1, I, d, expert_std(d), seed, threads)
    w["up_q"], w["up_s"] = gen_mxfp4(st, MAT_UP, 0, E + 1, I, d, expert_std(d), seed, threads)
    w["down_q"], w["down_s"] = gen_mxfp4(st, MAT_DOWN, 0, E + 1, d, I, expert_std(I), seed, threads)
    _EXPERT_CACHE[key] = w
    return w


Q2K_BLOCK_BYTES = 84  # bytes per 256-value Q2_K super-block
MAT_Q2K = 16            # stream families of Q2_K matrices: MAT_Q2K + MAT_GATE/UP/DOWN


def gen_q2k(set_tag: int, mat_tag: int, first: int, count: int, rows: int, K: int, std: float, seed: int = 0,
            threads=None) -> np.ndarray:
    out = np.empty((count, rows, K // 256 * Q2K_BLOCK_BYTES), dtype=np.uint8)
    rc = _load().synth_q2k(seed, set_tag, mat_tag, first, count, rows, K, std, _ptr(out), threads or usable_cpus())
    if rc != 0:
        raise ValueError("synth_q2k: bad shape")
    return out


_Q2K_CACHE = {}


def gen_experts_q2k(shape: MoEShape, seed: int = 0, threads=None) -> dict:
    """Routed experts 0..E-1 as Q2_K super-blocks: gate/up [E][I][d/256*84], down [E][d][I/256*84] (uint8);
    entries ~N(0, 1/sqrt(fan_in)) before quantisation, like the MXFP4 experts.  Cached per process."""
    key = (shape.weight_set, shape.n_experts, shape.d_model, shape.d_ff, seed)
    if key in _Q2K_CACHE:
        return _Q2K_CACHE[key]
    st = _set_tag(shape)
    E, d, I = shape.n_experts, shape.d_model, shape.d_ff
    w = {"gate": gen_q2k(st, MAT_Q2K + MAT_GATE, 0, E, I, d, expert_std(d), seed, threads),
         "up": gen_q2k(st, MAT_Q2K + MAT_UP, 0, E, I, d, expert_std(d), seed, threads),
         "down": gen_q2k(st, MAT_Q2K + MAT_DOWN, 0, E, d, I, expert_std(I), seed, threads)}
    _Q2K_CACHE[key] = w
    return w


def encode_q2k(v: np.ndarray) -> np.ndarray:
    """Encode fp32 rows [R][K] (K % 256 == 0) to Q2_K super-blocks [R][K/256*84]."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    R, K = v.shape
    assert K % 256 == 0
    out = np.empty((R, K // 256 * Q2K_BLOCK_BYTES), dtype=np.uint8)
    _load().synth_encode_q2k(_ptr(v), R, K, _ptr(out))
    return out


def encode_mxfp4(v: np.ndarray):
    """Encode fp32 rows [R][K] to MXFP4 (q [R][K/2], s [R][K/32])."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    R, K = v.shape
    assert K % 32 == 0
    q = np.empty((R, K // 2), dtype=np.uint8)
    s = np.empty((R, K // 32), dtype=np.uint8)
    _load().synth_encode_mxfp4(_ptr(v), R, K, _ptr(q), _ptr(s))
    return q, s


def gen_tid2eid(shape: MoEShape, seed: int = 0, threads=None) -> np.ndarray:
    out = np.empty((shape.vocab, shape.top_k), dtype=np.int32)
    rc = _load().synth_tid2eid(seed, _set_tag(shape), shape.vocab, shape.n_experts, shape.top_k,
                               _ptr(out), threads or usable_cpus())
    if rc != 0:
        raise ValueError("synth_tid2eid: bad shape")
    return out


def gen_token_ids(shape: MoEShape, seed: int = 0) -> np.ndarray:
    out = np.empty(shape.n_rows, dtype=np.int32)
    _load().synth_token_ids(seed, _cfg_tag(shape), shape.n_rows, shape.vocab, _ptr(out))
    return out


def gen_permutation(n: int, tag: int, seed: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.int32)
    _load().synth_permutation(seed, tag, n, _ptr(out))
    return out


def zipf_targets(shape: MoEShape, s: float = 1.2, seed: int = 0) -> np.ndarray:
    """Per-row selection probability per expert, q_e = min(1, c*rank_e^-s), sum q = k.

    A row picks k distinct experts, so no expert can hold more than 1/k of the
    assignments; capping q at 1 and filling the rest by rank is the closest
    Zipf-shaped load that k-of-E selection can reach.
    """
    E, k = shape.n_experts, shape.top_k
    ranks = np.arange(1, E + 1, dtype=np.float64)
    base = ranks ** (-s)
    lo, hi = 0.0, 1.0
    while np.minimum(1.0, hi * base).sum() < k:
        hi *= 2.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if np.minimum(1.0, mid * base).sum() < k:
            lo = mid
        else:
            hi = mid
    q_rank = np.minimum(1.0, hi * base)
    order = gen_permutation(E, 0x7A00 + _cfg_tag(shape), seed)  # rank i -> expert order[i]
    q = np.empty(E, dtype=np.float64)
    q[order] = q_rank
    return q


def resample_rows(shape: MoEShape, accept_rows, seed: int = 0, max_tries: int = 1000, threads=None,
                  with_index: bool = False):
    """Draw x and redraw every row that the filter rejects.

    `accept_rows(x_rows) -> bool[len(x_rows)]` (with_index: `accept_rows(x_rows,
    row_indices)`) is called on the rows drawn in each round (all rows first,
    then only the redrawn ones).  A rejected row r moves to its next attempt (a
    fresh stream of the same seed), so the accepted x is a function of the seed
    and the filter only.  Returns (x, attempts).
    """
    attempts = np.zeros(shape.n_rows, dtype=np.int32)
    x = gen_x(shape, seed, attempts, threads)
    todo = np.arange(shape.n_rows)
    for _ in range(max_tries):
        ok = np.asarray(accept_rows(x[todo], todo) if with_index else accept_rows(x[todo]), dtype=bool)
        todo = todo[~ok]
        if todo.size == 0:
            return x, attempts
        attempts[todo] += 1
        x = gen_x(shape, seed, attempts, threads)
    raise RuntimeError(f"{shape.name}: rows still rejected after {max_tries} redraws")


# Streams of the input-RMSNorm extras and the selection-only bias (numpy generators keyed by
# seed, workload and tensor).
_TAG_ROW_EXP, _TAG_NORM_W, _TAG_RESIDUAL, _TAG_SEL_BIAS, _TAG_SHARED_BF16 = 11, 12, 13, 14, 15


def _rng(shape: MoEShape, seed: int, tag: int):
    return np.random.default_rng(np.random.SeedSequence([seed, _cfg_tag(shape), tag]))


def bf16_bits(v) -> np.ndarray:
    """fp64/fp32 values -> bf16 bit patterns (via fp32, round to nearest even; finite inputs)."""
    u = np.ascontiguousarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def gen_row_exponents(shape: MoEShape, seed: int = 0) -> np.ndarray:
    """Per-row power-of-two scale exponents in [-3, 3] for the input-RMSNorm workloads."""
    return _rng(shape, seed, _TAG_ROW_EXP).integers(-3, 4, shape.n_rows).astype(np.int32)


def scale_rows_bf16(x_bits: np.ndarray, exps: np.ndarray) -> np.ndarray:
    """bf16 rows times 2^exps[r] (exact while in range)."""
    f = (x_bits.astype(np.uint32) << 16).view(np.float32) * np.ldexp(np.float32(1), exps)[:, None].astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def gen_norm_weight(shape: MoEShape, seed: int = 0) -> np.ndarray:
    """RMSNorm weight [d] as bf16 bits: 1 + N(0, 0.1)."""
    return bf16_bits(1.0 + 0.1 * _rng(shape, seed, _TAG_NORM_W).standard_normal(shape.d_model))


def gen_residual(shape: MoEShape, seed: int = 0) -> np.ndarray:
    """Residual rows [N][d] as bf16 bits: N(0, 1)."""
    return bf16_bits(_rng(shape, seed, _TAG_RESIDUAL).standard_normal((shape.n_rows, shape.d_model)))


def gen_selection_bias(shape: MoEShape, seed: int = 0) -> np.ndarray:
    """Router bias [E] fp32, N(0, 0.05), for the selection-only bias reading."""
    return (0.05 * _rng(shape, seed, _TAG_SEL_BIAS).standard_normal(shape.n_experts)).astype(np.float32)


def gen_shared_bf16(shape: MoEShape, seed: int = 0) -> dict:
    """A shared expert with bf16 weights, bf16 bit patterns: gate/up [I][d] ~ N(0, 1/sqrt(d)),
    down [d][I] ~ N(0, 1/sqrt(I)) (the routed experts' distributions before quantisation)."""
    g = _rng(shape, seed, _TAG_SHARED_BF16)
    d, I = shape.d_model, shape.d_ff
    return dict(gate=bf16_bits(expert_std(d) * g.standard_normal((I, d))),
                up=bf16_bits(expert_std(d) * g.standard_normal((I, d))),
                down=bf16_bits(expert_std(I) * g.standard_normal((d, I))))
