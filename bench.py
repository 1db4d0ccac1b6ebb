#!/usr/bin/env python3
"""Throughput of the routed MoE layer (sqrt-softplus top-6 of 256 + 1 shared
expert, MXFP4 SwiGLU experts) on one MI355X, through the C ABI.

One step = one moe_layer_forward over one batch of token rows with every input
already resident in HBM: activation split, router logits, top-k selection,
routing bookkeeping, gate/up GEMM, down GEMM, combine.  Default workload: the
512-row DSpark verify step (64 requests x 8 rows), d=4096, I=2048.

Prints one JSON line (rank 0).  Besides the contract fields it carries
- roofline: the gate/up GEMM (the dominant kernel) against HBM bandwidth, its
  duration measured with HIP events recorded on the launch stream around that
  kernel in every timed step;
- cpu_baseline: the fp64 CPU oracle timed on a bounded sample of the same
  workload on this host (routing of all rows, outputs of the first rows).
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
EXPERT_BYTES_NOTE = "gate+up MXFP4 bytes of every touched expert (incl. shared) + x and h at 2 B/value"
EXPERT_BYTES_NOTE_BF16 = ("gate+up MXFP4 bytes of every touched routed expert + the bf16 shared gate/up matrices "
                          "+ x and h at 2 B/value (two kernels: routed grouped GEMM and bf16 shared GEMM)")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gateup_verify512_traffic.txt")


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="verify512")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-sample-rows", type=int, default=512)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--shared-bf16", action="store_true",
                    help="the shared expert in bf16 (its own bf16-MFMA GEMMs) instead of MXFP4")
    ap.add_argument("--with-norm", action="store_true",
                    help="run the layer with its input RMSNorm and a residual add (seeded bf16 weight and residual)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one elementwise kernel over 1 GiB (reads 1 GiB, writes 1 GiB: the reference "
                         "for the HBM byte counters)")
    return ap.parse_args()


# hipEventDisableSystemFence: the event's record skips the system-scope cache
# write-back and invalidation, which would otherwise cost stream time at each
# record and slow the kernel that follows.  The events are read only after a
# device synchronisation.
HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000


class Hip:
    """The few HIP runtime calls the benchmark needs for events."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        ev = ctypes.c_void_p()
        if self.lib.hipEventCreateWithFlags(ctypes.byref(ev), HIP_EVENT_DISABLE_SYSTEM_FENCE) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        return ev.value

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        if self.lib.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, ev):
        self.lib.hipEventDestroy(ctypes.c_void_p(ev))


def kernel_source_digest():
    h = hashlib.sha256()
    for name in ("k_expert.hip", "common.h", "kernels.h"):
        with open(os.path.join(ROOT, "mxfp4_routed_expert_sqrt_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic(workload):
    """HBM bytes per gate/up launch from the committed counter summary, if it still matches the kernel."""
    if workload != "verify512" or not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            parts = line.split()
            if len(parts) == 2 and not line.startswith("#"):
                vals[parts[0]] = parts[1]
    if vals.get("kernel_source_digest") != kernel_source_digest():
        return None
    try:
        return int(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(shape, x, router_w, experts, rows, bias=None, token_ids=None, tid2eid=None):
    import oracle
    from mxfp4_routed_expert_sqrt_amd.synth import usable_cpus
    threads = usable_cpus()
    sample = list(range(min(rows, shape.n_rows)))
    # repeated until at least 10 s of CPU work (at most 3 passes) so that the rate is not a single short run
    passes, t0 = 0, time.perf_counter()
    while passes < 3 and (passes == 0 or time.perf_counter() - t0 < 10.0):
        oracle.forward(shape, x, router_w, experts, router_bias=bias, token_ids=token_ids, tid2eid=tid2eid,
                       rows=sample, threads=threads)
        passes += 1
    dt = time.perf_counter() - t0
    return {"value": passes * len(sample) / dt, "unit": "rows/s", "cores": threads, "kind": "oracle",
            "sample": f"fp64 oracle on rows 0..{len(sample) - 1} of the {shape.n_rows}-row {shape.name} batch "
                      f"(routing of all {shape.n_rows} rows, every touched expert decoded once), same inputs, "
                      f"{passes} pass(es); {dt:.1f} s wall"}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (expert parallelism is a design "
              "note only); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from mxfp4_routed_expert_sqrt_amd import capi, synth
    from mxfp4_routed_expert_sqrt_amd.configs import SHAPES
    from mxfp4_routed_expert_sqrt_amd.layer import MoELayer

    shape = SHAPES[args.workload]
    if shape.bias != "none":
        raise SystemExit(f"{shape.name} needs a calibrated router bias; benchmark a top-k or hash workload")
    dev = torch.device("cuda:0")
    t_gen = time.perf_counter()
    x_np = synth.gen_x(shape, args.seed)
    w_np = synth.gen_router(shape, args.seed)
    experts = synth.gen_experts(shape, args.seed)
    tok_np = tab_np = None
    if shape.routing == "hash":
        tok_np, tab_np = synth.gen_token_ids(shape, args.seed), synth.gen_tid2eid(shape, args.seed)
    print(f"[bench] inputs generated in {time.perf_counter() - t_gen:.1f}s", file=sys.stderr, flush=True)

    norm_w = resid = None
    if args.with_norm:
        norm_w = synth.gen_norm_weight(shape, args.seed)
        resid = torch.from_numpy(synth.gen_residual(shape, args.seed).view(np.int16)).to(dev).view(torch.bfloat16)
    shared_bf16 = synth.gen_shared_bf16(shape, args.seed) if args.shared_bf16 else None
    layer = MoELayer(shape, w_np, experts, dev, norm_w=norm_w, shared_bf16=shared_bf16)
    x = torch.from_numpy(x_np.view(np.int16)).to(dev).view(torch.bfloat16)
    tok = None if tok_np is None else torch.from_numpy(tok_np).to(dev)
    tab = None if tab_np is None else torch.from_numpy(tab_np).to(dev)
    out = torch.empty_like(x)
    ws = layer.new_workspace(shape.n_rows)

    # routing of this batch (untimed): touched experts for the byte count
    _, routing = layer.forward(x, tok, tab, with_routing=True, residual=resid)
    torch.cuda.synchronize()
    counts = routing["counts"].cpu().numpy()
    touched = int((counts > 0).sum()) + 1  # + shared expert
    N, d, I, E = shape.n_rows, shape.d_model, shape.d_ff, shape.n_experts
    per_expert = 3 * (I * d // 2 + I * d // 32)
    if args.shared_bf16:  # the grouped kernels then carry the routed experts only
        layer_bytes = (touched - 1) * per_expert + 3 * I * d * 2 + E * d * 4 + 2 * N * d * 2
        # the gate/up stage then times two kernels: the routed grouped GEMM and the bf16 shared GEMM
        gateup_bytes = ((touched - 1) * 2 * (I * d // 2 + I * d // 32) + N * d * 2 + N * shape.top_k * I * 2
                        + 2 * I * d * 2 + N * I * 2)
    else:
        layer_bytes = touched * per_expert + E * d * 4 + 2 * N * d * 2
        gateup_bytes = touched * 2 * (I * d // 2 + I * d // 32) + N * d * 2 + (N * shape.top_k + N) * I * 2

    hip = Hip()
    stream = torch.cuda.current_stream(dev).cuda_stream
    K, W = args.steps, args.warmup
    call = layer.args(x, out, ws, tok, tab, residual=resid)
    G = capi.STAGE_NAMES.index("gateup")

    def step(ev=None):
        call.stage_events = ctypes.cast(ev, ctypes.c_void_p) if ev is not None else None
        rc = capi.moe_layer_forward(layer.cfg, call, stream)
        if rc != capi.MOE_OK:
            raise capi.MoeError(rc)

    def event_array(evs):
        return (ctypes.c_void_p * capi.MOE_N_STAGE_EVENTS)(*evs)

    # timed steps: the only events recorded are the two around the gate/up
    # kernel, in every EV_STRIDE-th step (each event record costs ~9 us of
    # stream time, so events in every step would slow the measured step)
    ev_stride = max(1, K // 8)
    sampled = list(range(0, K, ev_stride))
    gu_events = [(hip.event(), hip.event()) for _ in sampled]
    gu_arrays = {i: event_array([a if s == G else b if s == G + 1 else None for s in range(capi.MOE_N_STAGE_EVENTS)])
                 for i, (a, b) in zip(sampled, gu_events)}
    for _ in range(W):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(gu_arrays.get(i))
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    gateup_ms = np.array([hip.elapsed_ms(a, b) for a, b in gu_events])

    # per-stage breakdown (untimed steps with every stage event recorded)
    KB = min(K, 20)
    events = [[hip.event() for _ in range(capi.MOE_N_STAGE_EVENTS)] for _ in range(KB)]
    ev_arrays = [event_array(evs) for evs in events]
    for i in range(KB):
        step(ev_arrays[i])
    torch.cuda.synchronize()
    stage_ms = np.array([[hip.elapsed_ms(events[i][s], events[i][s + 1]) for s in range(capi.MOE_N_STAGES)]
                         for i in range(KB)])
    gpu_ms = np.array([hip.elapsed_ms(events[i][0], events[i][-1]) for i in range(KB)])
    for evs in events + [list(p) for p in gu_events]:
        for e in evs:
            hip.destroy(e)

    if args.copy_calibration:
        # one elementwise kernel that reads 1 GiB and writes 1 GiB (a device copy may go to a DMA engine,
        # whose traffic the per-kernel counters do not see)
        src = torch.zeros(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.bitwise_not(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    ms_per_step = elapsed * 1e3 / K
    stages_us = {n: round(float(np.mean(stage_ms[:, s])) * 1e3, 2) for s, n in enumerate(capi.STAGE_NAMES)}
    t_gateup = float(np.mean(gateup_ms)) * 1e-3
    achieved = gateup_bytes / t_gateup / 1e9
    traffic = None if args.shared_bf16 else recorded_traffic(shape.name)
    result = {
        "metric": "MoE-layer token rows/s at 512-row verify" if shape.name == "verify512"
        else f"MoE-layer token rows/s ({shape.name})",
        "value": N / (ms_per_step * 1e-3),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # expert GEMM operands: FP4 weights x two-term FP8 activations, or FP6 terms on batches of tall
        # work units (at least 32 routed rows per expert on average, as the library chooses)
        "dtype": "fp4xfp6" if (N * shape.top_k >= 32 * E and I % 256 == 0 and d % 512 == 0) else "fp4xfp8",
        "data": "synthetic",
        "config": {"workload": f"{shape.name}: {N} token rows, d={d}, {E} routed experts top-{shape.top_k} + 1 "
                               f"shared, I={I}, MXFP4 experts ({shape.routing} routing)"
                               + (", input RMSNorm + residual add" if args.with_norm else "")
                               + (", bf16 shared expert" if args.shared_bf16 else ""),
                   "global_batch": N, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "gateup_kernel" + (" + shared_bf16_kernel<2>" if args.shared_bf16 else ""),
                     "algorithmic_bytes": gateup_bytes,
                     "bytes_definition": EXPERT_BYTES_NOTE_BF16 if args.shared_bf16 else EXPERT_BYTES_NOTE,
                     "kernel_us": t_gateup * 1e6,
                     "kernel_timing": f"HIP events around the gate/up kernel in {len(sampled)} of the {K} timed steps"},
        "layer": {"algorithmic_bytes": layer_bytes, "hbm_frac": layer_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
                  "touched_experts": touched, "stages_us": stages_us,
                  "stages_note": "separate untimed steps with an event before every stage (each event adds a few us)",
                  "gpu_us_per_step_with_stage_events": float(np.mean(gpu_ms)) * 1e3},
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle baseline", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(shape, x_np, w_np, experts, args.cpu_sample_rows,
                                              token_ids=tok_np, tid2eid=tab_np)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
