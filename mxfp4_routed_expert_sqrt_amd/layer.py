"""Thin torch-side wrapper of the C ABI: torch supplies device memory and the
stream, every step of the layer runs in the HIP library.
"""
import numpy as np
import torch

from . import capi
from .configs import MoEShape


def _ptr(t):
    return None if t is None else t.data_ptr()


def make_config(shape: MoEShape, has_shared: bool = True, route_scale=None, swiglu_limit=None,
                norm_eps: float = 1e-6, bias_mode: int = capi.MOE_BIAS_LOGIT,
                shared_format: int = capi.MOE_SHARED_MXFP4,
                expert_format: int = capi.MOE_EXPERTS_MXFP4) -> capi.MoeConfig:
    return capi.MoeConfig(shape.d_model, shape.d_ff, shape.n_experts, shape.top_k,
                          capi.MOE_ROUTING_TOPK if shape.routing == "topk" else capi.MOE_ROUTING_HASH,
                          1 if has_shared else 0,
                          float(shape.route_scale if route_scale is None else route_scale),
                          float(shape.swiglu_limit if swiglu_limit is None else swiglu_limit), float(norm_eps),
                          int(bias_mode), int(shared_format), int(expert_format))


def pack_mxfp4(q: torch.Tensor, s: torch.Tensor, rows: int, K: int, stream=None, out=None):
    """Natural-layout device tensors q [n][rows][K/2], s [n][rows][K/32] -> packed (q, s) device tensors.

    out: optional (q_out, s_out) uint8 device tensors of the packed sizes to pack into.
    """
    n = q.shape[0]
    qb, sb = capi.moe_packed_mxfp4_bytes(rows, K)
    if out is None:
        q_out = torch.empty(n * qb, dtype=torch.uint8, device=q.device)
        s_out = torch.empty(n * sb, dtype=torch.uint8, device=q.device)
    else:
        q_out, s_out = out
        assert q_out.numel() == n * qb and s_out.numel() == n * sb
    st = torch.cuda.current_stream(q.device).cuda_stream if stream is None else stream
    rc = capi.moe_pack_mxfp4(q.data_ptr(), s.data_ptr(), n, rows, K, q_out.data_ptr(), s_out.data_ptr(), st)
    if rc != capi.MOE_OK:
        raise capi.MoeError(rc)
    return q_out, s_out


def pack_q2k(q: torch.Tensor, rows: int, K: int, stream=None, out=None) -> torch.Tensor:
    """Natural-layout Q2_K device tensor q [n][rows][K/256*84] -> packed device tensor (same size)."""
    n = q.shape[0]
    nbytes = n * capi.moe_q2k_bytes(rows, K)
    q_out = torch.empty(nbytes, dtype=torch.uint8, device=q.device) if out is None else out
    assert q_out.numel() == nbytes
    st = torch.cuda.current_stream(q.device).cuda_stream if stream is None else stream
    rc = capi.moe_pack_q2k(q.data_ptr(), n, rows, K, q_out.data_ptr(), st)
    if rc != capi.MOE_OK:
        raise capi.MoeError(rc)
    return q_out


_ALIGN = 2 << 20  # each packed region starts on a 2 MiB boundary inside one allocation


def pack_bf16(w: torch.Tensor, rows: int, K: int, stream=None, out=None) -> torch.Tensor:
    """bf16 bit patterns [n][rows][K] (int16/uint16 device tensor) -> the fragment order of moe_pack_bf16
    (uint8 device tensor of the same byte size, or written into out)."""
    n = w.numel() // (rows * K)
    if out is None:
        out = torch.empty(n * rows * K * 2, dtype=torch.uint8, device=w.device)
    st = torch.cuda.current_stream(w.device).cuda_stream if stream is None else stream
    rc = capi.moe_pack_bf16(w.data_ptr(), n, rows, K, out.data_ptr(), st)
    if rc != capi.MOE_OK:
        raise capi.MoeError(rc)
    return out


class PackedExperts:
    """Routed experts 0..E-1 and the shared expert (index E), packed on the device.

    All packed matrices live in one device allocation, each region 2 MiB
    aligned, so the weight stream has the same placement from run to run.
    """

    def __init__(self, experts: dict, shape: MoEShape, device, has_shared: bool = True):
        E, d, I = shape.n_experts, shape.d_model, shape.d_ff
        mats = (("gate", I, d), ("up", I, d), ("down", d, I))
        regions, total = {}, 0
        for name, rows, K in mats:
            qb, sb = capi.moe_packed_mxfp4_bytes(rows, K)
            for key, count in ((name, E), ("sh_" + name, 1 if has_shared else 0)):
                if count == 0:
                    continue
                for part, nbytes in (("q", count * qb), ("s", count * sb)):
                    regions[(key, part)] = (total, nbytes)
                    total += (nbytes + _ALIGN - 1) // _ALIGN * _ALIGN
        self._regions, self._total = regions, total
        self._alloc(device)
        for name, rows, K in mats:
            q = torch.from_numpy(np.ascontiguousarray(experts[name + "_q"])).to(device)
            s = torch.from_numpy(np.ascontiguousarray(experts[name + "_s"])).to(device)
            self.t[name] = pack_mxfp4(q[:E], s[:E], rows, K, out=self.t[name])
            if has_shared:
                self.t["sh_" + name] = pack_mxfp4(q[E:E + 1], s[E:E + 1], rows, K, out=self.t["sh_" + name])
            del q, s
        torch.cuda.synchronize(device)
        self.has_shared = has_shared

    def _alloc(self, device):
        """One allocation with every region on a 2 MiB boundary; self.t = (q, s) views per matrix set."""
        self.buffer = torch.empty(self._total + _ALIGN, dtype=torch.uint8, device=device)
        self._base = (-self.buffer.data_ptr()) % _ALIGN
        view = lambda key, part: self.buffer[self._base + self._regions[(key, part)][0]:][:self._regions[(key, part)][1]]
        self.t = {key: (view(key, "q"), view(key, "s")) for key, part in self._regions if part == "q"}

    def copy(self) -> "PackedExperts":
        """A second device copy of the same packed weights (its own allocation, same 2 MiB placement)."""
        c = object.__new__(PackedExperts)
        c._regions, c._total, c.has_shared = self._regions, self._total, self.has_shared
        c._alloc(self.buffer.device)
        c.buffer[c._base:c._base + self._total].copy_(self.buffer[self._base:self._base + self._total])
        return c

    def weights(self, with_shared: bool = True, shared_bf16=None) -> capi.MoeWeights:
        """shared_bf16: optional dict of bf16 device tensors gate/up [I][d], down [d][I] (the shared expert
        in bf16; the packed MXFP4 shared expert is then not passed)."""
        t = self.t
        mx = self.has_shared and with_shared and shared_bf16 is None
        sh = (lambda n, i: _ptr(t["sh_" + n][i])) if mx else (lambda n, i: None)
        b = shared_bf16 or {}
        return capi.MoeWeights(_ptr(t["gate"][0]), _ptr(t["gate"][1]), _ptr(t["up"][0]), _ptr(t["up"][1]),
                               _ptr(t["down"][0]), _ptr(t["down"][1]), sh("gate", 0), sh("gate", 1), sh("up", 0),
                               sh("up", 1), sh("down", 0), sh("down", 1), _ptr(b.get("gate")), _ptr(b.get("up")),
                               _ptr(b.get("down")))


class PackedQ2kExperts:
    """Routed experts 0..E-1 in Q2_K, packed on the device (gate, up, down), one allocation."""

    def __init__(self, experts_q2k: dict, shape: MoEShape, device):
        E, d, I = shape.n_experts, shape.d_model, shape.d_ff
        mats = (("gate", I, d), ("up", I, d), ("down", d, I))
        sizes = {n: E * capi.moe_q2k_bytes(rows, K) for n, rows, K in mats}
        offs, total = {}, 0
        for n, _, _ in mats:
            offs[n] = total
            total += (sizes[n] + _ALIGN - 1) // _ALIGN * _ALIGN
        self.buffer = torch.empty(total + _ALIGN, dtype=torch.uint8, device=device)
        base = (-self.buffer.data_ptr()) % _ALIGN
        self.t = {}
        for n, rows, K in mats:
            view = self.buffer[base + offs[n]:][:sizes[n]]
            q = torch.from_numpy(np.ascontiguousarray(experts_q2k[n][:E])).to(device)
            self.t[n] = pack_q2k(q, rows, K, out=view)
            del q
        torch.cuda.synchronize(device)

    def weights(self, shared_bf16=None) -> capi.MoeWeights:
        b = shared_bf16 or {}
        t = self.t
        return capi.MoeWeights(_ptr(t["gate"]), None, _ptr(t["up"]), None, _ptr(t["down"]), None,
                               None, None, None, None, None, None,
                               _ptr(b.get("gate")), _ptr(b.get("up")), _ptr(b.get("down")))


class MoELayer:
    def __init__(self, shape: MoEShape, router_w, experts, device="cuda", router_bias=None,
                 has_shared: bool = True, route_scale=None, swiglu_limit=None, norm_w=None, norm_eps: float = 1e-6,
                 bias_mode: int = capi.MOE_BIAS_LOGIT, shared_bf16=None, experts_q2k=None, shared_stream: bool = True):
        """experts: natural-layout arrays (dict, packed here) or an already packed PackedExperts.
        norm_w: optional bf16 bit patterns [d] of the input RMSNorm weight (the layer then normalises x).
        shared_bf16: optional dict of bf16 bit patterns gate/up [I][d], down [d][I]: the shared expert in
        bf16 (MOE_SHARED_BF16) instead of the MXFP4 shared expert at index E of experts.
        experts_q2k: optional natural-layout Q2_K routed experts (dict gate/up/down, packed here) or a
        PackedQ2kExperts (MOE_EXPERTS_Q2K); experts is then not used, and the shared expert, if any,
        must be given in bf16."""
        self.shape = shape
        self.device = torch.device(device)
        fmt = capi.MOE_SHARED_MXFP4 if shared_bf16 is None else capi.MOE_SHARED_BF16
        if shared_bf16 is not None:
            has_shared = True
        efmt = capi.MOE_EXPERTS_MXFP4 if experts_q2k is None else capi.MOE_EXPERTS_Q2K
        if experts_q2k is not None and shared_bf16 is None and has_shared:
            raise ValueError("Q2_K routed experts take a bf16 shared expert (shared_bf16) or none (has_shared=False)")
        self.cfg = make_config(shape, has_shared, route_scale, swiglu_limit, norm_eps, bias_mode, fmt, efmt)
        self.shared_bf16 = None if shared_bf16 is None else {
            n: torch.from_numpy(np.ascontiguousarray(shared_bf16[n], dtype=np.uint16).view(np.int16)).to(self.device)
            for n in ("gate", "up", "down")}
        # the bf16 shared expert also packed into MFMA fragments (moe_args_t.sh_packed): gate, up, down back
        # to back; the layer streams it for batches of at least MOE_SHARED_STREAM_ROWS rows.  shared_stream
        # False keeps the LDS-tiled kernels at every size.
        self.sh_packed = None
        if self.shared_bf16 is not None and shared_stream:
            d, I = shape.d_model, shape.d_ff
            self.sh_packed = torch.empty(3 * I * d * 2, dtype=torch.uint8, device=self.device)
            for i, (n, rows, K) in enumerate((("gate", I, d), ("up", I, d), ("down", d, I))):
                pack_bf16(self.shared_bf16[n], rows, K, out=self.sh_packed[i * I * d * 2:(i + 1) * I * d * 2])
            torch.cuda.synchronize(self.device)
        self.norm_w = None if norm_w is None else \
            torch.from_numpy(np.ascontiguousarray(norm_w, dtype=np.uint16).view(np.int16)).to(self.device)
        self.router_w = torch.as_tensor(np.ascontiguousarray(router_w, dtype=np.float32)).to(self.device)
        self.router_bias = None if router_bias is None else \
            torch.as_tensor(np.ascontiguousarray(router_bias, dtype=np.float32)).to(self.device)
        mx_shared = has_shared and shared_bf16 is None
        self.q2k = None
        if experts_q2k is not None:
            self.q2k = experts_q2k if isinstance(experts_q2k, PackedQ2kExperts) else \
                PackedQ2kExperts(experts_q2k, shape, self.device)
            self.experts = None
        elif isinstance(experts, PackedExperts):
            if mx_shared and not experts.has_shared:
                raise ValueError("packed experts carry no shared expert")
            self.experts = experts
        else:
            self.experts = PackedExperts(experts, shape, self.device, mx_shared)
        self.has_shared = has_shared

    def workspace_bytes(self, n_rows: int) -> int:
        return capi.moe_workspace_size(self.cfg, n_rows)

    def new_workspace(self, n_rows: int) -> torch.Tensor:
        return torch.empty(max(self.workspace_bytes(n_rows), 256), dtype=torch.uint8, device=self.device)

    def args(self, x, out, workspace, token_ids=None, tid2eid=None, routing=None, residual=None) -> capi.MoeArgs:
        N = x.shape[0]
        r = routing or {}
        return capi.MoeArgs(N, _ptr(x), _ptr(self.router_w), _ptr(self.router_bias), _ptr(token_ids), _ptr(tid2eid),
                            0 if tid2eid is None else tid2eid.shape[0],
                            self.q2k.weights(self.shared_bf16) if self.q2k is not None else
                            self.experts.weights(self.has_shared, self.shared_bf16), _ptr(out),
                            _ptr(r.get("topk_idx")), _ptr(r.get("topk_w")), _ptr(r.get("counts")),
                            _ptr(r.get("offsets")), _ptr(r.get("perm")), _ptr(r.get("inv")), _ptr(workspace),
                            0 if workspace is None else workspace.numel(), None, _ptr(self.norm_w), _ptr(residual),
                            _ptr(self.sh_packed))

    def forward(self, x: torch.Tensor, token_ids=None, tid2eid=None, out=None, workspace=None, with_routing=False,
                stream=None, residual=None):
        """x: bf16 [N][d] on the device; residual: optional bf16 [N][d] added to the output.
        Returns out (bf16 [N][d]) or (out, routing dict)."""
        N, k, E = x.shape[0], self.shape.top_k, self.shape.n_experts
        if out is None:
            out = torch.empty_like(x)
        if workspace is None:
            workspace = self.new_workspace(N)
        routing = None
        if with_routing:
            dev = self.device
            routing = dict(topk_idx=torch.empty((N, k), dtype=torch.int32, device=dev),
                           topk_w=torch.empty((N, k), dtype=torch.float32, device=dev),
                           counts=torch.empty(E, dtype=torch.int32, device=dev),
                           offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
                           perm=torch.empty(N * k, dtype=torch.int32, device=dev),
                           inv=torch.empty(N * k, dtype=torch.int32, device=dev))
        st = torch.cuda.current_stream(self.device).cuda_stream if stream is None else stream
        rc = capi.moe_layer_forward(self.cfg, self.args(x, out, workspace, token_ids, tid2eid, routing, residual), st)
        if rc != capi.MOE_OK:
            raise capi.MoeError(rc)
        return (out, routing) if with_routing else out
