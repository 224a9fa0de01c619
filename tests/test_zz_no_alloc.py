"""moe_forward_noalloc (the workspace is the library's own device array) against
moe_forward with a caller workspace, through the C ABI: every output bit-identical, on two
calls in a row whose second has a smaller batch, with and without xp."""
import pytest
import torch

import expert_routing_amd as moe
from synth import CONFIGS
from gpu_cases import gpu_inputs

pytestmark = pytest.mark.gpu

OUTS = ("topk_ids", "topk_w", "counts", "offsets", "dest_row", "row_src", "send_bytes",
        "n_dropped", "y", "y_sh")

CASES = {
    # decode-sized batch, DeepSeek-V3-style group-limited sigmoid routing over 64 experts
    "decode": (CONFIGS["dsv3_decode"].with_(h=1024, E=64, inter=256), (32, 8)),
    # shared expert and 4 virtual ranks, capacity drops
    "shared_ep_cap": (CONFIGS["dsv3_ep8"].with_(T=256, h=512, E=64, K=6, inter=256,
                                               shared_inter=192, n_ep=4, ep_rank=1,
                                               capacity_factor=1.0), (256, 96)),
    "f32": (CONFIGS["tiny_f32"], (64, 24)),
}


def _call(cfg, inp, noalloc, gather):
    p = moe.problem_from_config(cfg, T=inp["T"])
    b = moe.alloc_buffers(p, "cuda")
    t = dict(b)
    t.update(x=inp["x"], w_router=inp["w_router"], bias=inp["bias"], w13=inp["w13"],
             w2=inp["w2"], w13_sh=inp["w13_sh"], w2_sh=inp["w2_sh"])
    if gather:
        t["xp"] = None
    if noalloc:
        moe.moe_forward_noalloc(p, t)
    else:
        moe.moe_forward(p, t, b["ws"])
    torch.cuda.synchronize()
    return b


@pytest.mark.parametrize("gather", [False, True])
@pytest.mark.parametrize("name", list(CASES))
def test_noalloc_equals_forward(name, gather):
    cfg, sizes = CASES[name]
    for T in sizes:          # two calls in a row, the second smaller
        c = cfg.with_(T=T)
        print(f"[case] noalloc {name} T={T} gather={gather}", flush=True)
        inp = gpu_inputs(c)
        want = _call(c, inp, noalloc=False, gather=gather)
        got = _call(c, inp, noalloc=True, gather=gather)
        for k in OUTS:
            if want[k] is not None:
                assert torch.equal(want[k], got[k]), (name, T, k)
        R = int(want["offsets"][-1].item())
        assert torch.equal(want["yp"][:R], got["yp"][:R])
