"""fp64 CPU oracle of the routed MoE layer (ctypes wrapper of moe_oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg use it to check and time the HIP implementation; the product
path never imports it.  It shares no code with the HIP implementation: inputs
arrive as plain arrays (bf16 bit patterns, fp32, MXFP4 bytes in the natural
[rows][K/2] + [rows][K/32] layout, or Q2_K super-blocks [rows][K/256*84])
and results come back in fp64.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "libmoe_oracle.so")
_lib = None


def build() -> str:
    """Compile the oracle with the host C compiler (no GPU code involved)."""
    cmd = ["gcc", "-std=c99", "-O2", "-fPIC", "-shared", "-pthread", "-Wall", "-o", _LIB, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    return _LIB


class _Cfg(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int), ("d", ctypes.c_int), ("E", ctypes.c_int), ("k", ctypes.c_int),
                ("I", ctypes.c_int), ("routing", ctypes.c_int), ("route_scale", ctypes.c_double),
                ("swiglu_limit", ctypes.c_double), ("norm_eps", ctypes.c_float), ("bias_mode", ctypes.c_int),
                ("expert_format", ctypes.c_int)]


class _Inputs(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("router_w", ctypes.c_void_p), ("router_bias", ctypes.c_void_p),
                ("token_ids", ctypes.c_void_p), ("tid2eid", ctypes.c_void_p), ("vocab", ctypes.c_long)] + \
               [(n, ctypes.c_void_p) for n in ("gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s",
                                              "sh_gate_q", "sh_gate_s", "sh_up_q", "sh_up_s", "sh_down_q",
                                              "sh_down_s", "norm_w", "residual", "sh_gate_w", "sh_up_w",
                                              "sh_down_w")]


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        vp, i32, dbl = ctypes.c_void_p, ctypes.c_int, ctypes.c_double
        lib.orc_e2m1.argtypes, lib.orc_e2m1.restype = [i32], dbl
        lib.orc_e8m0.argtypes, lib.orc_e8m0.restype = [i32], dbl
        lib.orc_bf16.argtypes, lib.orc_bf16.restype = [ctypes.c_uint16], dbl
        lib.orc_f32_to_bf16.argtypes, lib.orc_f32_to_bf16.restype = [ctypes.c_float], ctypes.c_uint16
        lib.orc_rmsnorm_bf16.argtypes = [vp, i32, i32, vp, ctypes.c_float, vp]
        lib.orc_decode_mxfp4_row.argtypes = [vp, vp, i32, vp]
        lib.orc_decode_q2k_row.argtypes = [vp, i32, vp]
        lib.orc_half.argtypes, lib.orc_half.restype = [ctypes.c_uint16], dbl
        lib.orc_router_logits.argtypes = [vp, i32, i32, vp, i32, vp, vp, i32]
        lib.orc_softplus.argtypes, lib.orc_softplus.restype = [dbl], dbl
        lib.orc_score.argtypes, lib.orc_score.restype = [dbl], dbl
        lib.orc_topk.argtypes, lib.orc_topk.restype = [vp, i32, i32, vp], dbl
        lib.orc_route.argtypes = [vp, i32, i32, i32, i32, vp, vp, ctypes.c_long, vp, vp, vp, vp]
        lib.orc_route.restype = i32
        lib.orc_bookkeeping.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp]
        lib.orc_forward.argtypes = [ctypes.POINTER(_Cfg), ctypes.POINTER(_Inputs), vp, i32, vp, vp, vp, vp, vp,
                                    vp, vp, vp, vp, i32]
        lib.orc_forward.restype = i32
        _lib = lib
    return _lib


def _p(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _threads(n):
    """n, or the CPUs this process may use: its affinity mask capped by a cgroup v2 CPU quota."""
    if n:
        return int(n)
    cpus = len(os.sched_getaffinity(0))
    try:
        with open("/sys/fs/cgroup/cpu.max") as f:
            quota, period = f.read().split()[:2]
        if quota != "max":
            cpus = min(cpus, int(quota) // int(period))
    except (OSError, ValueError):
        pass
    return max(1, cpus)


def e2m1(code: int) -> float:
    return _load().orc_e2m1(int(code))


def e8m0(e: int) -> float:
    return _load().orc_e8m0(int(e))


def bf16(bits: int) -> float:
    return _load().orc_bf16(int(bits))


def decode_mxfp4(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Decode an MXFP4 matrix q [R][K/2], s [R][K/32] to fp64 [R][K], one row at a time."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    s = np.ascontiguousarray(s, dtype=np.uint8)
    R, K = q.shape[0], q.shape[1] * 2
    out = np.empty((R, K), dtype=np.float64)
    lib = _load()
    for r in range(R):
        lib.orc_decode_mxfp4_row(_p(q[r]), _p(s[r]), K, _p(out[r]))
    return out


def half(bits: int) -> float:
    return _load().orc_half(int(bits))


def decode_q2k(blocks: np.ndarray, K: int) -> np.ndarray:
    """Decode a Q2_K matrix [R][K/256*84] (GGUF Q2_K super-blocks) to fp64 [R][K], one row at a time."""
    blocks = np.ascontiguousarray(blocks, dtype=np.uint8)
    R = blocks.shape[0]
    assert blocks.shape[1] == K // 256 * 84
    out = np.empty((R, K), dtype=np.float64)
    lib = _load()
    for r in range(R):
        lib.orc_decode_q2k_row(_p(blocks[r]), K, _p(out[r]))
    return out


def softplus(z: float) -> float:
    return _load().orc_softplus(float(z))


def score(z: float) -> float:
    return _load().orc_score(float(z))


def router_logits(x_bf16: np.ndarray, w: np.ndarray, bias=None, threads=None) -> np.ndarray:
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, d = x.shape
    E = w.shape[0]
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    z = np.empty((N, E), dtype=np.float64)
    _load().orc_router_logits(_p(x), N, d, _p(w), E, _p(b), _p(z), _threads(threads))
    return z


def topk(s: np.ndarray, k: int):
    """(ascending ids of the k largest scores, gap between k-th and (k+1)-th)."""
    s = np.ascontiguousarray(s, dtype=np.float64)
    idx = np.empty(k, dtype=np.int32)
    gap = _load().orc_topk(_p(s), s.shape[0], k, _p(idx))
    return idx, gap


def route(z: np.ndarray, k: int, routing: str = "topk", token_ids=None, tid2eid=None, sel_bias=None):
    """(idx [N][k] ascending, gates [N][k], margin [N]) from logits z [N][E].
    sel_bias: optional [E] added to the scores for the selection only."""
    z = np.ascontiguousarray(z, dtype=np.float64)
    N, E = z.shape
    idx = np.empty((N, k), dtype=np.int32)
    gates = np.empty((N, k), dtype=np.float64)
    margin = np.empty(N, dtype=np.float64)
    mode = 0 if routing == "topk" else 1
    tok = None if token_ids is None else np.ascontiguousarray(token_ids, dtype=np.int32)
    tab = None if tid2eid is None else np.ascontiguousarray(tid2eid, dtype=np.int32)
    vocab = 0 if tab is None else tab.shape[0]
    sb = None if sel_bias is None else np.ascontiguousarray(sel_bias, dtype=np.float32)
    rc = _load().orc_route(_p(z), N, E, k, mode, _p(tok), _p(tab), vocab, _p(sb), _p(idx), _p(gates), _p(margin))
    if rc != 0:
        raise ValueError("invalid hash-routing table entry")
    return idx, gates, margin


def bookkeeping(idx: np.ndarray, n_experts: int):
    """(counts [E], offsets [E+1], perm [N*k], inv [N*k]) of routing idx [N][k]."""
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    N, k = idx.shape
    counts = np.empty(n_experts, dtype=np.int32)
    offsets = np.empty(n_experts + 1, dtype=np.int32)
    perm = np.empty(N * k, dtype=np.int32)
    inv = np.empty(N * k, dtype=np.int32)
    _load().orc_bookkeeping(_p(idx), N, k, n_experts, _p(counts), _p(offsets), _p(perm), _p(inv))
    return counts, offsets, perm, inv


def rmsnorm_bf16(x_bf16: np.ndarray, g_bf16: np.ndarray, eps: float) -> np.ndarray:
    """bf16 [N][d] -> bf16 [N][d]: RMSNorm in fp32, one rounding (orc_rmsnorm_bf16)."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    g = np.ascontiguousarray(g_bf16, dtype=np.uint16)
    N, d = x.shape
    assert g.shape == (d,)
    out = np.empty_like(x)
    _load().orc_rmsnorm_bf16(_p(x), N, d, _p(g), float(eps), _p(out))
    return out


def forward(shape, x, router_w, experts, router_bias=None, token_ids=None, tid2eid=None, rows=None,
            route_scale=None, swiglu_limit=None, with_shared=True, threads=None, norm_w=None, norm_eps=1e-6,
            residual=None, bias_mode=0, shared_bf16=None, experts_q2k=None) -> dict:
    """The whole layer in fp64.

    bias_mode: 0 = router_bias added to the logits (selection and gates); 1 = added to the
    scores for the selection only (gates from the unbiased scores).

    norm_w: optional bf16 [d] RMSNorm weight; the layer then runs on rmsnorm_bf16(x, norm_w, norm_eps).
    residual: optional bf16 [N][d] added to the output.
    shared_bf16: optional dict of bf16 bit patterns gate/up [I][d], down [d][I]: the shared expert in
    bf16 (the MXFP4 shared expert at index E is then not used).
    experts_q2k: optional dict of Q2_K blocks gate/up [E][I][d/256*84], down [E][d][I/256*84]: the routed
    experts in Q2_K instead of the MXFP4 experts (whose shared expert, index E, still applies unless
    shared_bf16 is given or with_shared is False).

    experts: dict of natural-layout MXFP4 arrays gate_q/gate_s/up_q/up_s [E+1][I][...] and
    down_q/down_s [E+1][d][...]; index E is the shared expert (ignored if with_shared=False).
    rows: optional list of rows whose outputs are computed (routing always covers all rows).
    Returns out [n_out][d] fp64 and the full routing arrays.
    """
    N, d, E, k, I = shape.n_rows, shape.d_model, shape.n_experts, shape.top_k, shape.d_ff
    x = np.ascontiguousarray(x, dtype=np.uint16)
    assert x.shape == (N, d)
    cfg = _Cfg(N, d, E, k, I, 0 if shape.routing == "topk" else 1,
               float(shape.route_scale if route_scale is None else route_scale),
               float(shape.swiglu_limit if swiglu_limit is None else swiglu_limit), float(norm_eps), int(bias_mode),
               0 if experts_q2k is None else 1)
    keep = []

    def P(a, dtype=None):
        if a is None:
            return None
        a = np.ascontiguousarray(a, dtype=dtype) if dtype is not None else np.ascontiguousarray(a)
        keep.append(a)
        return a.ctypes.data

    w = experts
    mx_sh = with_shared and shared_bf16 is None
    b = shared_bf16 or {}
    if experts_q2k is not None:
        assert d % 256 == 0 and I % 256 == 0, "Q2_K experts need d and I multiples of 256"
        qk = experts_q2k
        routed = (P(qk["gate"][:E]), None, P(qk["up"][:E]), None, P(qk["down"][:E]), None)
    else:
        routed = (P(w["gate_q"][:E]), P(w["gate_s"][:E]), P(w["up_q"][:E]), P(w["up_s"][:E]),
                  P(w["down_q"][:E]), P(w["down_s"][:E]))
    ins = _Inputs(P(x), P(router_w, np.float32), P(router_bias, np.float32), P(token_ids, np.int32),
                  P(tid2eid, np.int32), 0 if tid2eid is None else int(np.asarray(tid2eid).shape[0]),
                  *routed,
                  P(w["gate_q"][E]) if mx_sh else None, P(w["gate_s"][E]) if mx_sh else None,
                  P(w["up_q"][E]) if mx_sh else None, P(w["up_s"][E]) if mx_sh else None,
                  P(w["down_q"][E]) if mx_sh else None, P(w["down_s"][E]) if mx_sh else None,
                  P(norm_w, np.uint16), P(residual, np.uint16), P(b.get("gate"), np.uint16),
                  P(b.get("up"), np.uint16), P(b.get("down"), np.uint16))
    rows_arr = None if rows is None else np.ascontiguousarray(rows, dtype=np.int32)
    n_out = N if rows_arr is None else rows_arr.shape[0]
    out = np.empty((n_out, d), dtype=np.float64)
    z = np.empty((N, E), dtype=np.float64)
    idx = np.empty((N, k), dtype=np.int32)
    gates = np.empty((N, k), dtype=np.float64)
    margin = np.empty(N, dtype=np.float64)
    counts = np.empty(E, dtype=np.int32)
    offsets = np.empty(E + 1, dtype=np.int32)
    perm = np.empty(N * k, dtype=np.int32)
    inv = np.empty(N * k, dtype=np.int32)
    rc = _load().orc_forward(ctypes.byref(cfg), ctypes.byref(ins), _p(rows_arr), n_out, _p(out), _p(z), _p(idx),
                             _p(gates), _p(margin), _p(counts), _p(offsets), _p(perm), _p(inv),
                             _threads(threads))
    if rc != 0:
        raise ValueError("invalid hash-routing table entry")
    return dict(out=out, z=z, idx=idx, gates=gates, margin=margin, counts=counts, offsets=offsets, perm=perm,
                inv=inv)
