"""An empty batch (T = 0) through the whole layer on the GPU: moe_forward returns MOE_OK
for every expert-weight format and router shape, and writes the layout of nothing: zero
counts, zero offsets, no dropped pairs and an all-zero send matrix. The oracle's dispatch
of zero tokens is the reference (every count of an empty token set is zero)."""
import numpy as np
import pytest
import torch

import expert_routing_amd as moe
import oracle
from synth import CONFIGS
from gpu_cases import gpu_inputs, np_, packed_weights
from test_gpu_mxfp8 import quantize_weights

pytestmark = pytest.mark.gpu

CASES = {
    # the fused small-expert-count router
    "fused_router": CONFIGS["mixtral_prefill"].with_(h=256, E=8, K=2, inter=256),
    # the tiled router, group-limited sigmoid scoring, 4 virtual ranks and a shared expert
    "shared_ep": CONFIGS["dsv3_ep8"].with_(h=256, E=32, K=4, n_groups=4, topk_groups=2,
                                          inter=128, shared_inter=128, n_ep=4, ep_rank=1),
    # capacity with padding to it
    "cap_pad": CONFIGS["mixtral_prefill"].with_(h=128, E=8, K=2, inter=128,
                                               capacity_factor=1.0, pad=True),
}


@pytest.mark.parametrize("fmt", ["bf16", "bf16_packed", "mxfp8"])
@pytest.mark.parametrize("name", list(CASES))
def test_empty_batch_forward(name, fmt):
    cfg = CASES[name]
    print(f"[case] empty {name} {fmt}", flush=True)
    inp = gpu_inputs(cfg, T=0)
    p = moe.problem_from_config(cfg, T=0, dtype="bf16_packed" if fmt == "bf16_packed" else None)
    if fmt == "mxfp8":
        p.act_dtype = moe.DTYPE["mxfp8"]
    b = moe.alloc_buffers(p, "cuda")
    for k in ("counts", "offsets", "n_dropped"):
        b[k].fill_(-7)
    if b["send_bytes"] is not None:
        b["send_bytes"].fill_(-7)
    t = dict(b)
    t.update(x=inp["x"], w_router=inp["w_router"], bias=inp["bias"], w13=inp["w13"],
             w2=inp["w2"], w13_sh=inp["w13_sh"], w2_sh=inp["w2_sh"], xp=None)
    if fmt == "bf16_packed":
        t.update(packed_weights(inp))
    if fmt == "mxfp8":
        for k in ("w13", "w2", "w13_sh", "w2_sh"):
            if inp[k] is None:
                t[k] = t[k + "_scale"] = None
                continue
            c, s = quantize_weights(inp[k].cpu())
            t[k] = torch.from_numpy(c).cuda()
            t[k + "_scale"] = torch.from_numpy(s).cuda()
    moe.moe_forward(p, t, b["ws"])   # raises on any status but MOE_OK
    torch.cuda.synchronize()
    d = oracle.dispatch(np.zeros((0, cfg.K), np.int64), E=cfg.E, n_ep=cfg.n_ep,
                        ep_rank=cfg.ep_rank, capacity_factor=cfg.capacity_factor, pad=cfg.pad,
                        h=cfg.h, dtype_size=cfg.act_bytes)
    np.testing.assert_array_equal(np_(b["counts"]), d.counts)
    np.testing.assert_array_equal(np_(b["offsets"]), d.offsets)
    assert int(np_(b["n_dropped"])[0]) == d.n_dropped == 0
    if b["send_bytes"] is not None:
        assert (np_(b["send_bytes"]) == 0).all()
