"""Full input sets of each workload, as the tests use them.

The two routing-dependent steps of the input recipe run here, with the oracle
making the routing decisions:
- rows whose top-k score margin (k-th minus (k+1)-th largest sqrt-softplus
  score, fp64, after any bias) is below 1e-3 are redrawn, so that the choice of
  experts cannot depend on rounding (all top-k workloads);
- the Zipf workload's logit bias is calibrated by 120 damped fixed-point steps
  b_e += 0.25 * (ln q_e - ln max(q_hat_e, 1/(2N))) on the workload's x, then
  frozen (undamped steps oscillate: the square root of the softplus compresses
  the score gaps of strongly biased experts).
"""
import functools
import time

import numpy as np

import oracle
from mxfp4_routed_expert_sqrt_amd import synth
from mxfp4_routed_expert_sqrt_amd.configs import SHAPES

MIN_MARGIN = 1e-3


ZIPF_STEPS, ZIPF_DAMPING = 120, 0.25


def calibrate_zipf_bias(shape, x, w, steps=ZIPF_STEPS, seed=0):
    q = synth.zipf_targets(shape, seed=seed)
    z0 = oracle.router_logits(x, w)
    b = np.zeros(shape.n_experts, dtype=np.float32)
    floor = 1.0 / (2 * shape.n_rows)
    for _ in range(steps):
        idx, _, _ = oracle.route(z0 + b.astype(np.float64)[None, :], shape.top_k)
        q_hat = np.bincount(idx.ravel(), minlength=shape.n_experts) / shape.n_rows
        b = (b.astype(np.float64) + ZIPF_DAMPING * (np.log(q) - np.log(np.maximum(q_hat, floor)))).astype(np.float32)
    return b, q


@functools.lru_cache(maxsize=None)
def workload(name, seed: int = 0, x_scale: float = 1.0):
    """dict(shape, x, router_w, bias, token_ids, tid2eid, experts, attempts).

    name: a workload name or a MoEShape.  x_scale (a power of two) multiplies
    the drawn x exactly before the margin filter (used to make the swiglu clamp bind).
    """
    shape = SHAPES[name] if isinstance(name, str) else name
    t0 = time.time()
    w = synth.gen_router(shape, seed)
    experts = synth.gen_experts(shape, seed)
    print(f"[inputs] {shape.name}: weights ready in {time.time() - t0:.1f}s", flush=True)
    bias = token_ids = tid2eid = None
    if shape.routing == "hash":
        x = synth.gen_x(shape, seed)
        attempts = np.zeros(shape.n_rows, dtype=np.int32)
        token_ids = synth.gen_token_ids(shape, seed)
        tid2eid = synth.gen_tid2eid(shape, seed)
    else:
        if shape.bias == "zipf":
            bias, _ = calibrate_zipf_bias(shape, synth.gen_x(shape, seed), w, seed=seed)

        def accept(rows):
            z = oracle.router_logits(rows, w, bias)
            _, _, margin = oracle.route(z, shape.top_k)
            return margin >= MIN_MARGIN

        if x_scale != 1.0:
            def accept_scaled(rows, _acc=accept):
                return _acc(_scale_bf16(rows, x_scale))
            x, attempts = synth.resample_rows(shape, accept_scaled, seed)
        else:
            x, attempts = synth.resample_rows(shape, accept, seed)
    if x_scale != 1.0:
        x = _scale_bf16(x, x_scale)
    print(f"[inputs] {shape.name}: x ready ({int((attempts > 0).sum())} rows redrawn) after "
          f"{time.time() - t0:.1f}s", flush=True)
    return dict(shape=shape, x=x, router_w=w, bias=bias, token_ids=token_ids, tid2eid=tid2eid,
                experts=experts, attempts=attempts)


NORM_EPS = 1e-6


@functools.lru_cache(maxsize=None)
def norm_workload(name, seed: int = 0):
    """The workload with the input RMSNorm and a residual: x rows drawn as usual, scaled by
    2^u per row (u in [-3, 3]), with the margin filter applied to RMSNorm(x); plus norm_w,
    norm_eps and residual."""
    base = workload(name, seed)
    shape = base["shape"]
    exps = synth.gen_row_exponents(shape, seed)
    g = synth.gen_norm_weight(shape, seed)

    def accept(rows, idx):
        xn = oracle.rmsnorm_bf16(synth.scale_rows_bf16(rows, exps[idx]), g, NORM_EPS)
        z = oracle.router_logits(xn, base["router_w"], base["bias"])
        _, _, margin = oracle.route(z, shape.top_k)
        return margin >= MIN_MARGIN

    if shape.routing == "hash":
        x, attempts = synth.gen_x(shape, seed), np.zeros(shape.n_rows, dtype=np.int32)
    else:
        x, attempts = synth.resample_rows(shape, accept, seed, with_index=True)
    wl = dict(base)
    wl.update(x=synth.scale_rows_bf16(x, exps), attempts=attempts, norm_w=g, norm_eps=NORM_EPS,
              residual=synth.gen_residual(shape, seed))
    return wl


@functools.lru_cache(maxsize=None)
def selection_bias_workload(name, seed: int = 0):
    """The workload with a router bias read as a selection-only bias (bias_mode 1): a seeded
    N(0, 0.05) fp32 bias added to the scores for choosing the experts; the margin filter runs on
    score + bias."""
    base = workload(name, seed)
    shape = base["shape"]
    bias = synth.gen_selection_bias(shape, seed)

    def accept(rows):
        z = oracle.router_logits(rows, base["router_w"])
        _, _, margin = oracle.route(z, shape.top_k, sel_bias=bias)
        return margin >= MIN_MARGIN

    x, attempts = synth.resample_rows(shape, accept, seed)
    wl = dict(base)
    wl.update(x=x, attempts=attempts, bias=bias, bias_mode=1)
    return wl


def _scale_bf16(x_bits, factor):
    """Multiply bf16 bit patterns by a power of two (exact while in range)."""
    f = (x_bits.astype(np.uint32) << 16).view(np.float32) * np.float32(factor)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def oracle_forward(wl, rows=None, **kw):
    if "bias_mode" in wl:
        kw.setdefault("bias_mode", wl["bias_mode"])
    if "norm_w" in wl:
        kw.setdefault("norm_w", wl["norm_w"])
        kw.setdefault("norm_eps", wl["norm_eps"])
        kw.setdefault("residual", wl["residual"])
    return oracle.forward(wl["shape"], wl["x"], wl["router_w"], wl["experts"], router_bias=wl["bias"],
                          token_ids=wl["token_ids"], tid2eid=wl["tid2eid"], rows=rows, **kw)
