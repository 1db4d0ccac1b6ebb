"""Full input sets of each workload, as the tests use them.

The two routing-dependent steps of the input recipe run here, with the oracle
making the routing decisions:
- rows whose top-k score margin (k-th minus (k+1)-th largest sqrt-softplus
  score, fp64, after any bias) is below 1e-3 are redrawn, so that the choice of
  experts cannot depend on rounding (all top-k workloads);
- the Zipf workload's logit bias is calibrated by 30 fixed-point steps
  b_e += ln q_e - ln max(q_hat_e, 1/(2N)) on the workload's x, then frozen.
"""
import functools

import numpy as np

import oracle
from mxfp4_routed_expert_sqrt_amd import synth
from mxfp4_routed_expert_sqrt_amd.configs import SHAPES

MIN_MARGIN = 1e-3


def calibrate_zipf_bias(shape, x, w, steps=30, seed=0):
    q = synth.zipf_targets(shape, seed=seed)
    z0 = oracle.router_logits(x, w)
    b = np.zeros(shape.n_experts, dtype=np.float32)
    floor = 1.0 / (2 * shape.n_rows)
    for _ in range(steps):
        idx, _, _ = oracle.route(z0 + b.astype(np.float64)[None, :], shape.top_k)
        q_hat = np.bincount(idx.ravel(), minlength=shape.n_experts) / shape.n_rows
        b = (b.astype(np.float64) + np.log(q) - np.log(np.maximum(q_hat, floor))).astype(np.float32)
    return b, q


@functools.lru_cache(maxsize=None)
def workload(name: str, seed: int = 0):
    """dict(shape, x, router_w, bias, token_ids, tid2eid, experts, attempts)."""
    shape = SHAPES[name]
    w = synth.gen_router(shape, seed)
    experts = synth.gen_experts(shape, seed)
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

        x, attempts = synth.resample_rows(shape, accept, seed)
    return dict(shape=shape, x=x, router_w=w, bias=bias, token_ids=token_ids, tid2eid=tid2eid,
                experts=experts, attempts=attempts)


def oracle_forward(wl, rows=None, **kw):
    return oracle.forward(wl["shape"], wl["x"], wl["router_w"], wl["experts"], router_bias=wl["bias"],
                          token_ids=wl["token_ids"], tid2eid=wl["tid2eid"], rows=rows, **kw)
