"""moe_layer_forward_noalloc: the layer on the library's static device scratch.

Through the C ABI: its output and routing are bitwise those of
moe_layer_forward with a caller workspace, on two calls in a row (the second
with a smaller batch, which takes other work-unit sizes over the scratch the
first call left behind); and it rejects what it cannot take (a workspace
argument, a batch beyond the scratch) before anything runs.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from mxfp4_routed_expert_sqrt_amd import capi, synth  # noqa: E402
from mxfp4_routed_expert_sqrt_amd.configs import SHAPES, MoEShape  # noqa: E402
from mxfp4_routed_expert_sqrt_amd.layer import MoELayer, make_config  # noqa: E402

V4 = SHAPES["verify512"]


def _host_rejects(cfg, n_rows, workspace=None):
    a = capi.MoeArgs()
    a.n_rows = n_rows
    a.x, a.router_w, a.out = 0x10000000, 0x20000000, 0x30000000
    w = capi.MoeWeights()
    for i, name in enumerate(n for n, _ in capi.MoeWeights._fields_):
        setattr(w, name, 0x100000000 + i * 0x100000000)
    a.w = w
    if workspace:
        a.workspace, a.workspace_bytes = workspace, 1 << 30
    return capi.moe_layer_forward_noalloc(cfg, a, None)


def test_noalloc_rejects_on_the_host():
    cfg = make_config(V4)
    n_max = 1
    while capi.moe_workspace_size(cfg, n_max + 1) <= capi.MOE_NOALLOC_SCRATCH_BYTES:
        n_max += 1
    assert n_max >= V4.n_rows  # the 512-row verify batch fits
    assert _host_rejects(cfg, n_max + 1) == capi.MOE_ERR_SCRATCH
    assert _host_rejects(cfg, 512, workspace=0x80000000) == capi.MOE_ERR_INVALID
    assert _host_rejects(cfg, -1) == capi.MOE_ERR_INVALID
    assert _host_rejects(cfg, 0) == capi.MOE_OK
    bad = make_config(V4)
    bad.top_k = 9
    assert _host_rejects(bad, 8) == capi.MOE_ERR_UNSUPPORTED
    assert "static scratch" in capi.moe_status_string(capi.MOE_ERR_SCRATCH)


def _run(layer, x, with_ws):
    N, k, E = x.shape[0], layer.shape.top_k, layer.shape.n_experts
    dev = x.device
    out = torch.empty_like(x)
    r = dict(topk_idx=torch.empty((N, k), dtype=torch.int32, device=dev),
             topk_w=torch.empty((N, k), dtype=torch.float32, device=dev),
             counts=torch.empty(E, dtype=torch.int32, device=dev),
             offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
             perm=torch.empty(N * k, dtype=torch.int32, device=dev),
             inv=torch.empty(N * k, dtype=torch.int32, device=dev))
    ws = layer.new_workspace(N) if with_ws else None
    args = layer.args(x, out, ws, routing=r)
    stream = torch.cuda.current_stream(dev).cuda_stream
    fn = capi.moe_layer_forward if with_ws else capi.moe_layer_forward_noalloc
    rc = fn(layer.cfg, args, stream)
    assert rc == capi.MOE_OK, capi.moe_status_string(rc)
    torch.cuda.synchronize()
    res = {key: v.cpu().numpy() for key, v in r.items()}
    res["out"] = out.view(torch.int16).cpu().numpy()
    return res


@pytest.mark.gpu
@pytest.mark.parametrize("shape,small", [(V4, 96), (MoEShape("edge_tall", 611, 512, 8, 4, 256, "topk", "edge_tall"), 37)],
                         ids=["verify512-then-96", "tall611-then-37"])
def test_noalloc_matches_the_workspace_entry_point(shape, small):
    dev = torch.device("cuda")
    print(f"noalloc {shape.name}: {shape.n_rows} rows then {small}", flush=True)
    layer = MoELayer(shape, synth.gen_router(shape), synth.gen_experts(shape), dev)
    x = torch.from_numpy(synth.gen_x(shape).view(np.int16)).to(dev).view(torch.bfloat16)
    for n in (shape.n_rows, small):  # the second call is smaller, on the scratch the first one left
        got = _run(layer, x[:n].contiguous(), with_ws=False)
        ref = _run(layer, x[:n].contiguous(), with_ws=True)
        for key in ref:
            assert np.array_equal(got[key], ref[key]), f"{shape.name} n={n}: {key} differs"
        print(f"noalloc {shape.name} n={n}: bitwise equal to moe_layer_forward", flush=True)
