"""ctypes binding of include/moe_mxfp4.h (argument marshalling only).

Every entry point has the same name and arguments as in the C header; device
pointers are passed as integers (e.g. torch's `data_ptr()`), the stream as a
hipStream_t integer (e.g. `torch.cuda.current_stream().cuda_stream`).  Loading
fails loudly if the HIP library has not been built: there is no fallback.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_mxfp4.so")

MOE_OK, MOE_ERR_INVALID, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 0, -1, -2, -3, -4
MOE_ERR_SCRATCH = -5
MOE_NOALLOC_SCRATCH_BYTES = 96 << 20
MOE_ROUTING_TOPK, MOE_ROUTING_HASH = 0, 1
MOE_BIAS_LOGIT, MOE_BIAS_SELECT = 0, 1
MOE_SHARED_MXFP4, MOE_SHARED_BF16 = 0, 1
MOE_EXPERTS_MXFP4, MOE_EXPERTS_Q2K = 0, 1
Q2K_BLOCK_BYTES = 84  # one 256-value Q2_K super-block
MOE_MAX_ROWS = 1 << 20
MOE_SHARED_STREAM_ROWS = 2048

c_i32, c_i64, c_f32, c_vp, c_size = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t


class MoeConfig(ctypes.Structure):
    _fields_ = [("d_model", c_i32), ("d_ff", c_i32), ("n_experts", c_i32), ("top_k", c_i32), ("routing", c_i32),
                ("has_shared", c_i32), ("route_scale", c_f32), ("swiglu_limit", c_f32), ("norm_eps", c_f32),
                ("bias_mode", c_i32), ("shared_format", c_i32), ("expert_format", c_i32)]


class MoeWeights(ctypes.Structure):
    _fields_ = [(n, c_vp) for n in ("gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s", "sh_gate_q", "sh_gate_s",
                                    "sh_up_q", "sh_up_s", "sh_down_q", "sh_down_s", "sh_gate_w", "sh_up_w",
                                    "sh_down_w")]


class MoeArgs(ctypes.Structure):
    _fields_ = [("n_rows", c_i32), ("x", c_vp), ("router_w", c_vp), ("router_bias", c_vp), ("token_ids", c_vp),
                ("tid2eid", c_vp), ("vocab", c_i64), ("w", MoeWeights), ("out", c_vp), ("topk_idx", c_vp),
                ("topk_w", c_vp), ("counts", c_vp), ("offsets", c_vp), ("perm", c_vp), ("inv", c_vp),
                ("workspace", c_vp), ("workspace_bytes", c_size), ("stage_events", c_vp), ("norm_w", c_vp),
                ("residual", c_vp), ("sh_packed", c_vp)]


MOE_N_STAGES = 5
MOE_N_STAGE_EVENTS = MOE_N_STAGES + 1
STAGE_NAMES = ("router", "select_route", "gateup", "down", "combine")


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library {LIB_PATH} is not built (run __graft_entry__.build()); "
                               "there is no CPU fallback")
        L = ctypes.CDLL(LIB_PATH)
        L.moe_version.argtypes, L.moe_version.restype = [], ctypes.c_int
        L.moe_status_string.argtypes, L.moe_status_string.restype = [ctypes.c_int], ctypes.c_char_p
        L.moe_packed_mxfp4_bytes.argtypes = [c_i32, c_i32, ctypes.POINTER(c_size), ctypes.POINTER(c_size)]
        L.moe_packed_mxfp4_bytes.restype = ctypes.c_int
        L.moe_pack_mxfp4.argtypes = [c_vp, c_vp, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp]
        L.moe_pack_mxfp4.restype = ctypes.c_int
        L.moe_q2k_bytes.argtypes = [c_i32, c_i32, ctypes.POINTER(c_size)]
        L.moe_q2k_bytes.restype = ctypes.c_int
        L.moe_pack_q2k.argtypes = [c_vp, c_i32, c_i32, c_i32, c_vp, c_vp]
        L.moe_pack_q2k.restype = ctypes.c_int
        L.moe_pack_bf16.argtypes = [c_vp, c_i32, c_i32, c_i32, c_vp, c_vp]
        L.moe_pack_bf16.restype = ctypes.c_int
        L.moe_workspace_size.argtypes = [ctypes.POINTER(MoeConfig), c_i32, ctypes.POINTER(c_size)]
        L.moe_workspace_size.restype = ctypes.c_int
        L.moe_layer_forward.argtypes = [ctypes.POINTER(MoeConfig), ctypes.POINTER(MoeArgs), c_vp]
        L.moe_layer_forward.restype = ctypes.c_int
        L.moe_layer_forward_noalloc.argtypes = [ctypes.POINTER(MoeConfig), ctypes.POINTER(MoeArgs), c_vp]
        L.moe_layer_forward_noalloc.restype = ctypes.c_int
        _lib = L
    return _lib


EXPORTED = ("moe_version", "moe_status_string", "moe_packed_mxfp4_bytes", "moe_pack_mxfp4", "moe_q2k_bytes",
            "moe_pack_q2k", "moe_pack_bf16", "moe_workspace_size", "moe_layer_forward", "moe_layer_forward_noalloc")


class MoeError(RuntimeError):
    def __init__(self, status):
        self.status = status
        super().__init__(f"moe status {status}: {moe_status_string(status)}")


def _check(status):
    if status != MOE_OK:
        raise MoeError(status)
    return status


def moe_version() -> int:
    return lib().moe_version()


def moe_status_string(status: int) -> str:
    return lib().moe_status_string(status).decode()


def moe_packed_mxfp4_bytes(rows: int, K: int):
    q, s = c_size(), c_size()
    _check(lib().moe_packed_mxfp4_bytes(rows, K, ctypes.byref(q), ctypes.byref(s)))
    return q.value, s.value


def moe_pack_mxfp4(q, s, n_mat, rows, K, q_out, s_out, stream) -> int:
    return lib().moe_pack_mxfp4(q, s, n_mat, rows, K, q_out, s_out, stream)


def moe_q2k_bytes(rows: int, K: int) -> int:
    b = c_size()
    _check(lib().moe_q2k_bytes(rows, K, ctypes.byref(b)))
    return b.value


def moe_pack_q2k(q, n_mat, rows, K, q_out, stream) -> int:
    return lib().moe_pack_q2k(q, n_mat, rows, K, q_out, stream)


def moe_pack_bf16(w, n_mat, rows, K, out, stream) -> int:
    return lib().moe_pack_bf16(w, n_mat, rows, K, out, stream)


def moe_workspace_size(cfg: MoeConfig, n_rows: int) -> int:
    b = c_size()
    _check(lib().moe_workspace_size(ctypes.byref(cfg), n_rows, ctypes.byref(b)))
    return b.value


def moe_layer_forward(cfg: MoeConfig, args: MoeArgs, stream) -> int:
    return lib().moe_layer_forward(ctypes.byref(cfg), ctypes.byref(args), stream)


def moe_layer_forward_noalloc(cfg: MoeConfig, args: MoeArgs, stream) -> int:
    return lib().moe_layer_forward_noalloc(ctypes.byref(cfg), ctypes.byref(args), stream)
