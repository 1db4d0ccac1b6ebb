#!/usr/bin/env python3
"""Throughput of the routed MoE layer (sqrt-softplus top-6 of 256 + 1 shared
expert, MXFP4 SwiGLU experts) on one MI355X, through the C ABI.

One step = one moe_layer_forward over one batch of token rows with every input
already resident in HBM: router logits and activation split, top-k selection,
routing bookkeeping, gate/up GEMM, down GEMM, combine.  Headline workload: the
512-row DSpark verify step (64 requests x 8 rows), d=4096, I=2048.

Protocol per workload: a pre-heat of layer calls for a fixed wall time (the
GPU's clocks settle), the W warm-up steps, then exactly K timed steps between
device synchronisations with no event recorded inside them (two HIP events on
the launch stream bracket the whole window as a cross-check).  Kernel
durations come from a separate loop of K steps after the timed window, with a
HIP event before every stage on the launch stream (each record adds stream
time between kernels, which is why they stay out of the timed steps).

Prints one JSON line.  Besides the contract fields it carries
- roofline: the dominant kernel (gate/up) against HBM bandwidth, its algorithmic
  bytes (gate+up MXFP4 bytes of every touched expert + x) over its duration;
  layer_frac: the whole layer's algorithmic bytes (touched experts' weights,
  router weight, x, out) over ms_per_step;
- workloads: the same measurement on the other layer configurations (8-row
  decode with four weight copies rotated, 8192-row prefill with its FP4-MFMA
  fraction, Zipf-skewed and hash-routed 2048-row batches) and on the drafter's
  expert format (Q2_K routed experts with a bf16 shared expert) at the
  448-row draft slab and the 512-row verify batch;
- cpu_baseline: the fp64 CPU oracle on a bounded sample of the headline
  workload on this host (all host cores, and one core on 8 rows);
- hbm_read_probe: the read bandwidth a plain streaming kernel reaches on this
  GPU (2 GiB read once per launch, regular and non-temporal loads, the best of
  four grid sizes), the practical ceiling beside the 8 TB/s data-sheet peak;
  roofline.peak_measured and frac_of_measured set the dominant kernel against
  it (roofline.peak stays the data-sheet figure).
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
FP4_PEAK_TFLOPS = 10100.0  # dense MXFP4 MFMA, MI355X
BF16_PEAK_TFLOPS = 2500.0  # dense bf16/fp16 MFMA, MI355X (the Q2_K GEMMs)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gateup_verify512_traffic.txt")
EXTRA_WORKLOADS = ("decode8", "prefill8192", "zipf2048", "hash2048", "q2k_draft448", "q2k_verify512")
Q2K_PREFIX = "q2k_"  # routed experts in Q2_K, shared expert in bf16, on the named shape
DECODE_WEIGHT_COPIES = 4  # 8-row batches touch ~0.6 GB of weights: rotate copies past the 256 MB MALL
HBM_PROBE_LIB = os.path.join(ROOT, "mxfp4_routed_expert_sqrt_amd", "libmoe_hbm.so")
HBM_PROBE_BYTES = 2 << 30  # 8x the 256 MB memory-side cache
HBM_PROBE_GRIDS = (2048, 4096, 8192, 16384)  # workgroups of 256 threads


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--preheat-s", type=float, default=1.0,
                    help="wall time of untimed layer calls before the warm-up steps of each workload")
    ap.add_argument("--workload", default="verify512", help="the headline workload")
    ap.add_argument("--only", action="store_true", help="measure the headline workload only")
    ap.add_argument("--extra", default=None,
                    help="comma-separated workloads to measure after the headline (default: all of "
                         + ", ".join(EXTRA_WORKLOADS) + ")")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-sample-rows", type=int, default=512)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--shared-bf16", action="store_true",
                    help="the shared expert in bf16 (its own bf16-MFMA GEMMs) instead of MXFP4")
    ap.add_argument("--with-norm", action="store_true",
                    help="run the layer with its input RMSNorm and a residual add (seeded bf16 weight and residual)")
    ap.add_argument("--no-hbm-probe", action="store_true",
                    help="skip the streaming-read probe (profiling runs of the layer's kernels)")
    ap.add_argument("--hbm-probe-only", action="store_true",
                    help="run only the streaming-read probe and print its JSON (for profiling it)")
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
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        ev = ctypes.c_void_p()
        if self.lib.hipEventCreateWithFlags(ctypes.byref(ev), HIP_EVENT_DISABLE_SYSTEM_FENCE) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        return ev.value

    def record(self, ev, stream):
        if self.lib.hipEventRecord(ctypes.c_void_p(ev), ctypes.c_void_p(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

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


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ---------------------------------------------------------------- byte model

def mxfp4_matrix_bytes(rows, K):
    return rows * K // 2 + rows * K // 32  # E2M1 nibbles + one E8M0 byte per 32 values


def q2k_matrix_bytes(rows, K):
    return rows * (K // 256) * 84  # one 84-byte super-block per 256 values


def algorithmic(shape, touched_routed, shared_bf16=False, has_bias=False, q2k=False):
    """Algorithmic HBM bytes and FP4-equivalent flops of the layer and its two GEMMs.

    Bytes: weights of every touched expert (an expert with no rows reads none) + router weight + x + out
    (+ bias, token ids and the rows' table entries in hash mode).  Intermediates (logits, h, y, index
    arrays) are implementation traffic, not algorithmic bytes.  Flops: 2 per multiply-add of the FP4
    weights (6*d*I per (row, expert): gate, up, down), whatever the activation format.
    """
    N, d, I, E, k = shape.n_rows, shape.d_model, shape.d_ff, shape.n_experts, shape.top_k
    m = (q2k_matrix_bytes if q2k else mxfp4_matrix_bytes)(I, d)  # gate, up [I][d] and down [d][I]: same size
    sh_mat = I * d * 2 if shared_bf16 else m
    x_bytes = out_bytes = N * d * 2
    extra = (E * 4 if has_bias else 0) + ((N * 4 + N * k * 4) if shape.routing == "hash" else 0)
    pairs = N * (k + 1)
    return {
        "layer_bytes": touched_routed * 3 * m + 3 * sh_mat + E * d * 4 + x_bytes + out_bytes + extra,
        "gateup_bytes": touched_routed * 2 * m + 2 * sh_mat + x_bytes,
        "down_bytes": touched_routed * m + sh_mat,
        "layer_flops": 6 * d * I * pairs,
        "gateup_flops": 4 * d * I * pairs,
        "down_flops": 2 * d * I * pairs,
    }


# ---------------------------------------------------------------- measurement

class Runner:
    """Runs one workload's layer calls on the current stream and times them."""

    def __init__(self, hip, layer, calls, stream):
        from mxfp4_routed_expert_sqrt_amd import capi
        self.capi, self.hip, self.layer, self.calls, self.stream = capi, hip, layer, calls, stream
        self.i = 0

    def step(self, events=None):
        call = self.calls[self.i % len(self.calls)]
        self.i += 1
        call.stage_events = events
        rc = self.capi.moe_layer_forward(self.layer.cfg, call, self.stream)
        call.stage_events = None
        if rc != self.capi.MOE_OK:
            raise self.capi.MoeError(rc)

    def run(self, K, W, preheat_s):
        import numpy as np
        import torch
        capi, hip = self.capi, self.hip
        # pre-heat for a fixed wall time, synchronising every 16 calls
        t0, n_pre = time.perf_counter(), 0
        while time.perf_counter() - t0 < preheat_s:
            for _ in range(16):
                self.step()
            n_pre += 16
            torch.cuda.synchronize()
        preheat = time.perf_counter() - t0
        for _ in range(W):
            self.step()
        torch.cuda.synchronize()
        ev0, ev1 = hip.event(), hip.event()
        t0 = time.perf_counter()
        hip.record(ev0, self.stream)
        for _ in range(K):
            self.step()
        hip.record(ev1, self.stream)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        gpu_ms = hip.elapsed_ms(ev0, ev1)
        # kernel durations: a separate loop of K steps with an event before every stage
        evs = [[hip.event() for _ in range(capi.MOE_N_STAGE_EVENTS)] for _ in range(K)]
        arrays = [(ctypes.c_void_p * capi.MOE_N_STAGE_EVENTS)(*e) for e in evs]
        for i in range(K):
            self.step(ctypes.cast(arrays[i], ctypes.c_void_p))
        torch.cuda.synchronize()
        stage_ms = np.array([[hip.elapsed_ms(e[s], e[s + 1]) for s in range(capi.MOE_N_STAGES)] for e in evs])
        for e in evs + [[ev0, ev1]]:
            for x in e:
                hip.destroy(x)
        # per-step spread: the sum of one step's stage intervals in that loop (p10, median, p90)
        step_us = stage_ms.sum(axis=1) * 1e3
        return {"preheat_s": preheat, "preheat_calls": n_pre, "ms_per_step": elapsed * 1e3 / K,
                "gpu_ms_per_step": gpu_ms / K,
                "stages_us": {n: float(np.mean(stage_ms[:, s])) * 1e3 for s, n in enumerate(capi.STAGE_NAMES)},
                "step_us_p10_p50_p90": [float(v) for v in np.percentile(step_us, [10, 50, 90])],
                "gateup_us_p10_p50_p90": [float(v) for v in np.percentile(stage_ms[:, capi.STAGE_NAMES.index("gateup")] * 1e3,
                                                                         [10, 50, 90])]}


def summarise(shape, timing, touched_routed, shared_bf16=False, has_bias=False, q2k=False):
    """Rates and roofline fractions; the MFMA fraction is against the FP4 peak (MXFP4 experts) or the bf16
    peak (Q2_K experts, whose GEMMs run on bf16/fp16 MFMA), under the key fp4_frac or bf16_frac."""
    a = algorithmic(shape, touched_routed, shared_bf16, has_bias, q2k)
    t = timing["ms_per_step"] * 1e-3
    gu, dn = timing["stages_us"]["gateup"] * 1e-6, timing["stages_us"]["down"] * 1e-6
    r = lambda v: round(v, 4)
    peak, fk = (BF16_PEAK_TFLOPS, "bf16_frac") if q2k else (FP4_PEAK_TFLOPS, "fp4_frac")
    return {
        "rows": shape.n_rows,
        "rows_per_s": shape.n_rows / t,
        "us_per_step": timing["ms_per_step"] * 1e3,
        "gpu_event_us_per_step": timing["gpu_ms_per_step"] * 1e3,
        "touched_experts": touched_routed + 1,
        "layer": {"algorithmic_bytes": a["layer_bytes"], "hbm_frac": r(a["layer_bytes"] / t / 1e9 / HBM_PEAK_GBS),
                  "flops": a["layer_flops"], fk: r(a["layer_flops"] / t / 1e12 / peak)},
        "gateup": {"us": timing["stages_us"]["gateup"], "algorithmic_bytes": a["gateup_bytes"],
                   "hbm_frac": r(a["gateup_bytes"] / gu / 1e9 / HBM_PEAK_GBS),
                   fk: r(a["gateup_flops"] / gu / 1e12 / peak)},
        "down": {"us": timing["stages_us"]["down"], "algorithmic_bytes": a["down_bytes"],
                 "hbm_frac": r(a["down_bytes"] / dn / 1e9 / HBM_PEAK_GBS),
                 fk: r(a["down_flops"] / dn / 1e12 / peak)},
        "stages_us": {k: round(v, 2) for k, v in timing["stages_us"].items()},
        # spread over the steps of the stage-timing loop (its events add a little stream time per step)
        "stage_loop_step_us_p10_p50_p90": [round(v, 1) for v in timing["step_us_p10_p50_p90"]],
        "gateup_us_p10_p50_p90": [round(v, 1) for v in timing["gateup_us_p10_p50_p90"]],
        "preheat_s": round(timing["preheat_s"], 3),
        "preheat_calls": timing["preheat_calls"],
    }


def cpu_baseline(shape, x, router_w, experts, rows, bias=None, token_ids=None, tid2eid=None):
    import numpy as np

    import oracle
    from mxfp4_routed_expert_sqrt_amd.synth import usable_cpus
    threads = usable_cpus()
    sample = list(range(min(rows, shape.n_rows)))
    # repeated until at least 10 s of CPU work (at most 3 passes) so that the rate is not a single short run
    passes, t0 = 0, time.perf_counter()
    while passes < 3 and (passes == 0 or time.perf_counter() - t0 < 10.0):
        ref = oracle.forward(shape, x, router_w, experts, router_bias=bias, token_ids=token_ids, tid2eid=tid2eid,
                             rows=sample, threads=threads)
        passes += 1
    dt = time.perf_counter() - t0
    # one core on 8 rows (the 8-row decode batch's size; every expert those rows touch decoded once)
    one = list(range(min(8, shape.n_rows)))
    t1 = time.perf_counter()
    oracle.forward(shape, x, router_w, experts, router_bias=bias, token_ids=token_ids, tid2eid=tid2eid, rows=one,
                   threads=1)
    dt1 = time.perf_counter() - t1
    # the oracle's rounding floor: what one bf16 rounding of its own output costs against the bar
    out = ref["out"]
    u = out.astype(np.float32).view(np.uint32)  # fp32 then bf16, each to nearest even, as the combine rounds
    rounded = (((u + np.uint32(0x7FFF) + ((u >> 16) & np.uint32(1))) >> 16) << 16).view(np.float32)
    err = np.abs(rounded.astype(np.float64) - out)
    return {"value": passes * len(sample) / dt, "unit": "rows/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"fp64 oracle on rows 0..{len(sample) - 1} of the {shape.n_rows}-row {shape.name} batch "
                      f"(routing of all {shape.n_rows} rows, every touched expert decoded once), same inputs, "
                      f"{passes} pass(es); {dt:.1f} s wall",
            "one_core": {"rows": len(one), "seconds": dt1, "rows_per_s": len(one) / dt1},
            "rounding_floor": {"max_err_over_rms": float(err.max() / np.sqrt(np.mean(out ** 2))),
                               "mean_rel": float(err.sum() / np.abs(out).sum())}}


# ---------------------------------------------------------------- workloads

def calibrate_zipf_bias(shape, layer, x, steps=120, damping=0.25, seed=0):
    """Logit bias that steers the per-row selection probability of expert e towards the Zipf(1.2) target
    q_e: b_e += 0.25 * (ln q_e - ln max(q_hat_e, 1/(2N))), q_hat from the layer's own counts, 120 steps,
    then frozen (the recipe of the parity tests, with the layer's routing in place of the oracle's)."""
    import numpy as np
    import torch

    from mxfp4_routed_expert_sqrt_amd import synth
    q = synth.zipf_targets(shape, seed=seed)
    floor = 1.0 / (2 * shape.n_rows)
    b = np.zeros(shape.n_experts, dtype=np.float32)
    for _ in range(steps):
        layer.router_bias.copy_(torch.from_numpy(b))
        _, routing = layer.forward(x, with_routing=True)
        q_hat = routing["counts"].cpu().numpy() / shape.n_rows
        b = (b.astype(np.float64) + damping * (np.log(q) - np.log(np.maximum(q_hat, floor)))).astype(np.float32)
    layer.router_bias.copy_(torch.from_numpy(b))
    torch.cuda.synchronize()
    return b


def measure_workload(name, ctx, args, hip):
    import numpy as np
    import torch

    from mxfp4_routed_expert_sqrt_amd import synth
    from mxfp4_routed_expert_sqrt_amd.configs import SHAPES
    from mxfp4_routed_expert_sqrt_amd.layer import MoELayer, PackedQ2kExperts

    q2k = name.startswith(Q2K_PREFIX)
    shape = SHAPES[name[len(Q2K_PREFIX):] if q2k else name]
    dev = ctx["dev"]
    x_np = synth.gen_x(shape, args.seed)
    x = torch.from_numpy(x_np.view(np.int16)).to(dev).view(torch.bfloat16)
    tok = tab = None
    if shape.routing == "hash":
        tok = torch.from_numpy(synth.gen_token_ids(shape, args.seed)).to(dev)
        tab = torch.from_numpy(synth.gen_tid2eid(shape, args.seed)).to(dev)
    bias = np.zeros(shape.n_experts, dtype=np.float32) if shape.bias == "zipf" else None
    note = None
    if q2k:
        if "q2k" not in ctx:
            t0 = time.perf_counter()
            ctx["q2k"] = PackedQ2kExperts(synth.gen_experts_q2k(shape, args.seed), shape, dev)
            ctx["shared_bf16"] = synth.gen_shared_bf16(shape, args.seed)
            print(f"[bench] Q2_K experts ready in {time.perf_counter() - t0:.1f}s", file=sys.stderr, flush=True)
        layer = MoELayer(shape, ctx["router_w"], None, dev, router_bias=bias, shared_bf16=ctx["shared_bf16"],
                         experts_q2k=ctx["q2k"])
        note = "routed experts in Q2_K (84 bytes per 256 values), shared expert in bf16"
    else:
        layer = MoELayer(shape, ctx["router_w"], ctx["packed"], dev, router_bias=bias)
    if shape.bias == "zipf":
        calibrate_zipf_bias(shape, layer, x, seed=args.seed)
    _, routing = layer.forward(x, tok, tab, with_routing=True)
    torch.cuda.synchronize()
    counts = routing["counts"].cpu().numpy()
    touched = int((counts > 0).sum())
    copies = [ctx["packed"]]
    if name == "decode8":
        while len(ctx["copies"]) < DECODE_WEIGHT_COPIES - 1:
            ctx["copies"].append(ctx["packed"].copy())
        copies += ctx["copies"]
        torch.cuda.synchronize()
        note = f"{len(copies)} device copies of the packed weights, used in turn"
    out = torch.empty_like(x)
    ws = layer.new_workspace(shape.n_rows)
    calls = []
    if q2k:
        calls.append(layer.args(x, out, ws, tok, tab))
    else:
        for c in copies:
            layer.experts = c
            calls.append(layer.args(x, out, ws, tok, tab))
        layer.experts = ctx["packed"]
    stream = torch.cuda.current_stream(dev).cuda_stream
    timing = Runner(hip, layer, calls, stream).run(args.steps, args.warmup, args.preheat_s)
    res = summarise(shape, timing, touched, shared_bf16=q2k, has_bias=bias is not None, q2k=q2k)
    if note:
        res["weights"] = note
    if shape.bias == "zipf":
        load = counts / shape.n_rows
        res["hottest_expert_share_of_assignments"] = round(float(load.max() / shape.top_k), 4)
    del ws, out
    return res


def hbm_read_peak(hip, dev, stream, reps=10, warm=3):
    """Read bandwidth of the streaming-read probe (libmoe_hbm.so) over HBM_PROBE_BYTES, per load kind."""
    import torch
    if not os.path.exists(HBM_PROBE_LIB):
        raise SystemExit(f"{HBM_PROBE_LIB} is missing: run __graft_entry__.build() first")
    lib = ctypes.CDLL(HBM_PROBE_LIB)
    lib.hbm_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
                                   ctypes.c_void_p]
    lib.hbm_probe_sink_words.argtypes = [ctypes.c_int]
    buf = torch.zeros(HBM_PROBE_BYTES, dtype=torch.uint8, device=dev)
    out = {"bytes_per_launch": HBM_PROBE_BYTES, "launches_timed": reps, "kernel": "hbm_read_kernel",
           "gbs_by_workgroups": {}}
    e0, e1 = hip.event(), hip.event()
    for nt, kind in ((0, "regular"), (1, "nontemporal")):
        per = {}
        for wg in HBM_PROBE_GRIDS:
            sink = torch.empty(lib.hbm_probe_sink_words(wg), dtype=torch.int32, device=dev)

            def call():
                if lib.hbm_read_probe(buf.data_ptr(), HBM_PROBE_BYTES, nt, sink.data_ptr(), wg, stream) != 0:
                    raise RuntimeError("hbm_read_probe failed")
            for _ in range(warm):
                call()
            torch.cuda.synchronize()
            hip.record(e0, stream)
            for _ in range(reps):
                call()
            hip.record(e1, stream)
            torch.cuda.synchronize()
            per[wg] = round(HBM_PROBE_BYTES * reps / (hip.elapsed_ms(e0, e1) * 1e-3) / 1e9, 1)
        out["gbs_by_workgroups"][kind] = per
        out[f"read_gbs_{kind}"] = max(per.values())
    hip.destroy(e0)
    hip.destroy(e1)
    out["read_gbs"] = max(out["read_gbs_regular"], out["read_gbs_nontemporal"])
    out["frac_of_spec"] = round(out["read_gbs"] / HBM_PEAK_GBS, 4)
    del buf
    return out


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (expert parallelism across GPUs is "
              "not implemented); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from mxfp4_routed_expert_sqrt_amd import synth
    from mxfp4_routed_expert_sqrt_amd.configs import SHAPES
    from mxfp4_routed_expert_sqrt_amd.layer import MoELayer, PackedExperts

    if args.hbm_probe_only:
        dev = torch.device("cuda:0")
        print(json.dumps({"hbm_read_probe": hbm_read_peak(Hip(), dev, torch.cuda.current_stream(dev).cuda_stream)}),
              flush=True)
        return

    shape = SHAPES[args.workload]
    if shape.bias != "none":
        raise SystemExit(f"{shape.name} needs a calibrated router bias: it runs in the workloads block")
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
    packed = PackedExperts(experts, shape, dev, True)
    layer = MoELayer(shape, w_np, packed, dev, norm_w=norm_w, shared_bf16=shared_bf16)
    x = torch.from_numpy(x_np.view(np.int16)).to(dev).view(torch.bfloat16)
    tok = None if tok_np is None else torch.from_numpy(tok_np).to(dev)
    tab = None if tab_np is None else torch.from_numpy(tab_np).to(dev)
    out = torch.empty_like(x)
    ws = layer.new_workspace(shape.n_rows)

    # routing of this batch (untimed): touched experts for the byte count
    _, routing = layer.forward(x, tok, tab, with_routing=True, residual=resid)
    torch.cuda.synchronize()
    touched = int((routing["counts"].cpu().numpy() > 0).sum())

    hip = Hip()
    stream = torch.cuda.current_stream(dev).cuda_stream
    K, W = args.steps, args.warmup
    print(f"[bench] {shape.name}: pre-heat {args.preheat_s:.1f}s, {W} warm-up, {K} timed steps", file=sys.stderr,
          flush=True)
    timing = Runner(hip, layer, [layer.args(x, out, ws, tok, tab, residual=resid)], stream).run(K, W, args.preheat_s)
    head = summarise(shape, timing, touched, shared_bf16=args.shared_bf16)

    if args.copy_calibration:
        # one elementwise kernel that reads 1 GiB and writes 1 GiB (a device copy may go to a DMA engine,
        # whose traffic the per-kernel counters do not see)
        src = torch.zeros(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.bitwise_not(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    probe = None
    if not args.no_hbm_probe:
        print("[bench] streaming-read probe", file=sys.stderr, flush=True)
        probe = hbm_read_peak(hip, dev, stream)

    N, d, I, E = shape.n_rows, shape.d_model, shape.d_ff, shape.n_experts
    ms_per_step = timing["ms_per_step"]
    gu = head["gateup"]
    achieved = gu["algorithmic_bytes"] / (gu["us"] * 1e-6) / 1e9
    traffic = None if (args.shared_bf16 or args.with_norm) else recorded_traffic(shape.name)
    result = {
        "metric": "MoE-layer token rows/s at 512-row verify" if shape.name == "verify512"
        else f"MoE-layer token rows/s ({shape.name})",
        "value": N / (ms_per_step * 1e-3),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "preheat_s": round(timing["preheat_s"], 3),
        "preheat_calls": timing["preheat_calls"],
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
                     "peak_measured": probe["read_gbs"] if probe else None,
                     "frac_of_measured": achieved / probe["read_gbs"] if probe else None,
                     "kernel": "gateup_kernel" + (" + shared_bf16_kernel<2>" if args.shared_bf16 else ""),
                     "algorithmic_bytes": gu["algorithmic_bytes"],
                     "bytes_definition": "gate+up MXFP4 bytes (nibbles + E8M0 scales) of every touched expert, "
                                         "incl. the shared one, + x (bf16)",
                     "kernel_us": gu["us"],
                     "kernel_timing": f"HIP events before every stage in a separate loop of {K} steps after the "
                                      "timed window, on the launch stream",
                     "layer_frac": head["layer"]["hbm_frac"],
                     "layer_bytes_definition": "MXFP4 weights of every touched expert + router weight fp32 + x + "
                                               "out (bf16), over ms_per_step"},
        "layer": head,
        "hbm_read_probe": probe,
    }
    if not args.only:
        ctx = {"dev": dev, "router_w": w_np, "packed": packed, "copies": []}
        result["workloads"] = {}
        extra = EXTRA_WORKLOADS if args.extra is None else tuple(w for w in args.extra.split(",") if w)
        for name in extra:
            if name not in EXTRA_WORKLOADS:
                raise SystemExit(f"unknown workload {name}; choose from {', '.join(EXTRA_WORKLOADS)}")
            if name == shape.name:
                continue
            print(f"[bench] workload {name}", file=sys.stderr, flush=True)
            result["workloads"][name] = measure_workload(name, ctx, args, hip)
        del ctx
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle baseline", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(shape, x_np, w_np, experts, args.cpu_sample_rows,
                                              token_ids=tok_np, tid2eid=tab_np)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
