"""Run-to-run and workspace robustness of the HIP path, through the C ABI.

The layer keeps no state between calls: every workspace region it reads is
written earlier in the same call.  These tests poison the workspace, reuse it
across calls of different sizes, record stage events with some entries left
NULL and replay a captured HIP graph of one call, and require
bitwise-identical outputs and routing.
"""
import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from mxfp4_routed_expert_sqrt_amd import capi  # noqa: E402
from mxfp4_routed_expert_sqrt_amd.configs import SHAPES, MoEShape  # noqa: E402
from mxfp4_routed_expert_sqrt_amd.layer import MoELayer, PackedExperts  # noqa: E402
from tests.inputs import workload  # noqa: E402

pytestmark = pytest.mark.gpu

TALL = MoEShape("edge_tall", 611, 512, 8, 4, 256, "topk", "edge_tall")
MEDIUM = MoEShape("edge_medium", 300, 512, 64, 4, 256, "topk", "edge_medium", bias="zipf")
# 1200 routed pairs at widths the wider units do not divide: the 16-row units of larger batches
WIDE16 = MoEShape("edge_w16_d768_i512", 300, 768, 64, 4, 512, "topk", "edge_w16b")
# 38 selection workgroups x 256 experts: the histogram bases go through global memory, scatter in-kernel
HISTG = MoEShape("edge_hist_global", 600, 256, 256, 6, 128, "topk", "edge_hist")


def _layer(wl):
    sh = wl["shape"]
    dev = torch.device("cuda")
    packed = PackedExperts(wl["experts"], sh, dev, True)
    return MoELayer(sh, wl["router_w"], packed, dev, router_bias=wl["bias"])


def _inputs(wl, rows=None):
    sh = wl["shape"]
    x = wl["x"] if rows is None else wl["x"][:rows]
    xt = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)
    tok = tab = None
    if sh.routing == "hash":
        ids = wl["token_ids"] if rows is None else wl["token_ids"][:rows]
        tok = torch.from_numpy(np.ascontiguousarray(ids)).cuda()
        tab = torch.from_numpy(wl["tid2eid"]).cuda()
    return xt, tok, tab


def _run(layer, x, tok, tab, ws):
    out, routing = layer.forward(x, tok, tab, workspace=ws, with_routing=True)
    torch.cuda.synchronize()
    res = {k: v.cpu().numpy() for k, v in routing.items()}
    res["out"] = out.view(torch.int16).cpu().numpy()
    return res


def _same(a, b, label):
    for key in a:
        assert np.array_equal(a[key], b[key]), f"{label}: {key} differs"


@pytest.mark.parametrize("shape", [TALL, MEDIUM, WIDE16, HISTG, SHAPES["hash2048"]],
                         ids=["tall", "medium", "wide16", "hist-global", "hash2048-scatter"])
def test_poisoned_workspace_repeatable(shape):
    # tall, medium: the 64- and 32-row work units; wide16: 16-row units of a batch of >= 1024 pairs;
    # hist-global: the selection's bases in global memory with the in-kernel scatter (medium bases
    # stay in LDS); hash2048: 12288 pairs, so the separate scatter launch
    wl = workload(shape)
    layer = _layer(wl)
    x, tok, tab = _inputs(wl)
    print(f"poisoned workspace {shape.name} N={shape.n_rows}", flush=True)
    ws = torch.full((layer.workspace_bytes(shape.n_rows),), 0xAB, dtype=torch.uint8, device="cuda")
    first = _run(layer, x, tok, tab, ws)
    ws.fill_(0x5C)
    second = _run(layer, x, tok, tab, ws)
    third = _run(layer, x, tok, tab, layer.new_workspace(shape.n_rows))
    _same(first, second, shape.name)
    _same(first, third, shape.name)


def test_workspace_reused_for_a_smaller_batch():
    wl = workload(TALL)
    layer = _layer(wl)
    big = layer.new_workspace(TALL.n_rows)
    x, tok, tab = _inputs(wl)
    _run(layer, x, tok, tab, big)  # leaves the big call's data in the workspace
    xs, toks, tabs = _inputs(wl, rows=100)
    print("workspace reuse: 611 rows, then 100 rows", flush=True)
    reused = _run(layer, xs, toks, tabs, big)
    fresh = _run(layer, xs, toks, tabs, layer.new_workspace(100))
    _same(reused, fresh, "reuse")


def test_residual_in_place_matches_separate_buffers():
    from tests.inputs import norm_workload
    wl = norm_workload("tiny")
    sh = wl["shape"]
    dev = torch.device("cuda")
    layer = MoELayer(sh, wl["router_w"], PackedExperts(wl["experts"], sh, dev, True), dev, norm_w=wl["norm_w"],
                     norm_eps=wl["norm_eps"])
    x, _, _ = _inputs(wl)
    resid = torch.from_numpy(wl["residual"].view(np.int16)).to(dev).view(torch.bfloat16)
    print("residual: separate buffer, then in place", flush=True)
    sep = layer.forward(x, residual=resid)
    inplace = resid.clone()
    layer.forward(x, out=inplace, residual=inplace)
    torch.cuda.synchronize()
    assert torch.equal(sep.view(torch.int16), inplace.view(torch.int16))
    plain = layer.forward(x)  # no residual: out differs from sep by the residual only
    torch.cuda.synchronize()
    assert not torch.equal(sep, plain)


def test_stage_events_with_null_entries():
    wl = workload("tiny")
    layer = _layer(wl)
    x, tok, tab = _inputs(wl)
    want = _run(layer, x, tok, tab, layer.new_workspace(x.shape[0]))
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    evs = []
    for _ in range(2):
        e = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
        evs.append(e.value)
    arr = (ctypes.c_void_p * capi.MOE_N_STAGE_EVENTS)(*([None] * capi.MOE_N_STAGE_EVENTS))
    g = capi.STAGE_NAMES.index("gateup")
    arr[g], arr[g + 1] = evs
    out = torch.empty_like(x)
    ws = layer.new_workspace(x.shape[0])
    call = layer.args(x, out, ws, tok, tab)
    call.stage_events = ctypes.cast(arr, ctypes.c_void_p)
    print("stage events: only the two around gate/up", flush=True)
    assert capi.moe_layer_forward(layer.cfg, call, torch.cuda.current_stream().cuda_stream) == capi.MOE_OK
    torch.cuda.synchronize()
    assert np.array_equal(out.view(torch.int16).cpu().numpy(), want["out"])
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    ms = ctypes.c_float()
    assert hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(evs[0]), ctypes.c_void_p(evs[1])) == 0
    assert ms.value > 0.0
    for e in evs:
        hip.hipEventDestroy(ctypes.c_void_p(e))


@pytest.mark.parametrize("name,bf16_shared", [("decode8", False), ("verify512", False), ("verify512", True)],
                         ids=["decode8", "verify512", "verify512-bf16shared"])
def test_graph_capture_replays_match_eager(name, bf16_shared):
    # The forward enqueues kernels only (no memsets, no host synchronisation), so
    # one call can be captured in a HIP graph.  Replays alternate two different
    # batches copied into the captured input buffer, with eager calls in between:
    # each must equal the eager result of its batch (no state carried over).
    from mxfp4_routed_expert_sqrt_amd import synth
    wls = [workload(name, seed) for seed in (0, 1)]
    sh = wls[0]["shape"]
    dev = torch.device("cuda")
    shared_bf16 = synth.gen_shared_bf16(sh) if bf16_shared else None
    layer = MoELayer(sh, wls[0]["router_w"], PackedExperts(wls[0]["experts"], sh, dev, True), dev,
                     router_bias=wls[0]["bias"], shared_bf16=shared_bf16)
    xs = [_inputs(w)[0] for w in wls]
    want = []
    for xb in xs:
        eager = layer.forward(xb, out=torch.empty_like(xb), workspace=layer.new_workspace(xb.shape[0]))
        torch.cuda.synchronize()
        want.append(eager.view(torch.int16).cpu().numpy())
    assert not np.array_equal(want[0], want[1])
    x = xs[0].clone()
    ws = layer.new_workspace(x.shape[0])
    out = torch.empty_like(x)
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):  # first call outside capture (one-time attribute setup)
        layer.forward(x, out=out, workspace=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    print(f"graph capture {name} bf16_shared={bf16_shared}", flush=True)
    with torch.cuda.graph(g, stream=side):
        layer.forward(x, out=out, workspace=ws)
    for i in range(4):
        out.zero_()
        x.copy_(xs[i % 2])
        layer.forward(xs[1 - i % 2], out=torch.empty_like(x), workspace=layer.new_workspace(x.shape[0]))  # eager work
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.view(torch.int16).cpu().numpy(), want[i % 2]), f"replay {i} differs"
