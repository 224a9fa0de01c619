"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI and bring
its results back, plus the error metrics the tolerances are stated in."""
from __future__ import annotations

import numpy as np
import torch

import expert_routing_amd as moe
from synth import make_inputs


def packed_weights(inp):
    """The expert weights of a bf16 workload in the packed order (moe_pack_weights)."""
    return {k: (None if inp[k] is None else moe.pack_weights(inp[k]))
            for k in ("w13", "w2", "w13_sh", "w2_sh")}


def run_stages(cfg, inp, p=None, packed=False):
    """route -> dispatch -> expert FFN -> combine, one ABI call per stage (packed: bf16
    with packed expert weights)."""
    p = p or moe.problem_from_config(cfg, T=inp["T"], dtype="bf16_packed" if packed else None)
    if packed:
        inp = dict(inp, **packed_weights(inp))
    b = moe.alloc_buffers(p, "cuda")
    if cfg.keys == "uniform":
        moe.moe_select(p, inp["keys"], inp["bias"], b["topk_ids"], b["topk_w"])
    else:
        moe.moe_route(p, inp["x"], inp["w_router"], inp["bias"], b["topk_ids"], b["topk_w"], b["ws"])
    x = inp.get("x")
    moe.moe_dispatch(p, x, b["topk_ids"], b["counts"], b["offsets"], b["dest_row"], b["row_src"],
                     b["send_bytes"], b["n_dropped"], b["xp"] if x is not None else None, b["ws"])
    if cfg.inter > 0 and x is not None:
        moe.moe_expert_ffn(p, b["xp"], b["offsets"], inp["w13"], inp["w2"], x, inp["w13_sh"],
                           inp["w2_sh"], b["yp"], b["y_sh"], b["ws"])
        moe.moe_combine(p, b["yp"], b["dest_row"], b["topk_w"], b["y_sh"], b["y"])
    torch.cuda.synchronize()
    return p, b


def run_forward(cfg, inp, p=None, gather=False, packed=False):
    """moe_forward; gather=True passes no xp, so the gate/up GEMM reads x through row_src;
    packed: bf16 with packed expert weights."""
    p = p or moe.problem_from_config(cfg, T=inp["T"], dtype="bf16_packed" if packed else None)
    if packed:
        inp = dict(inp, **packed_weights(inp))
    b = moe.alloc_buffers(p, "cuda")
    t = dict(b)
    t.update(x=inp["x"], w_router=inp["w_router"], bias=inp["bias"], w13=inp["w13"],
             w2=inp["w2"], w13_sh=inp["w13_sh"], w2_sh=inp["w2_sh"])
    if gather:
        t["xp"] = None
        b["xp"] = None
    moe.moe_forward(p, t, b["ws"])
    torch.cuda.synchronize()
    return p, b


def cpu_inputs(inp):
    return {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


def gpu_inputs(cfg, T=None):
    return make_inputs(cfg, device="cuda", T=T)


def np_(t):
    if t is None:
        return None
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy()


def rel_errors(got, ref):
    """(max_rel, mean_rel): max over rows of ||d||inf/||ref||inf (rows with ref != 0),
    and sum|d| / sum|ref|. Rows whose reference is exactly zero must match exactly."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    d = np.abs(got - ref)
    rmax = np.abs(ref).max(axis=1)
    nz = rmax > 0
    max_rel = float((d.max(axis=1)[nz] / rmax[nz]).max()) if nz.any() else 0.0
    zero_rows_exact = bool((d[~nz] == 0).all())
    mean_rel = float(d.sum() / max(np.abs(ref).sum(), 1e-300))
    return max_rel, mean_rel, zero_rows_exact


# Tolerances of the layer's outputs: fp32 runs 1e-4 relative; bf16 runs 2e-2 max-relative
# and 5e-3 mean-relative (fp32 accumulation, one bf16 rounding of the gated product and
# one of each output).
TOL = {"f32": (1e-4, 1e-4), "bf16": (2e-2, 5e-3)}
# Routing weights. From given fp32 logits (moe_select) only the kernels' exp, sigmoid and
# division round: a few ulp, so 1e-6 relative. From x (moe_route) the weights also carry
# the fp32 logits' accumulation error: a weight moves by at most 2 max_e |dL_e| relative
# (softmax over the selection, or sigmoid renormalised). The router's partial sums stay
# O(1) (x ~ N(0,1), W_r ~ N(0,1/h)), so a length-h fp32 sum errs by about u sqrt(h) in
# probability (u = 2^-24; 5e-6 at h = 7168), i.e. weights within ~1e-5; 1e-4 leaves a
# margin of ten for the tails over tens of thousands of weights.
W_RTOL_SELECT = 1e-6
W_RTOL = 1e-4


def routing_mismatches(ids_gpu, rr, tie=1e-4):
    """Tokens whose GPU id set differs from the oracle's, split into near-ties (K-th /
    (K+1)-th key gap or M-th / (M+1)-th group-score gap below `tie`) and others."""
    bad = np.nonzero((ids_gpu != rr.ids).any(axis=1))[0]
    near = (rr.kth_gap < tie) | (rr.group_gap < tie)
    return [int(t) for t in bad if near[t]], [int(t) for t in bad if not near[t]], int(near.sum())
