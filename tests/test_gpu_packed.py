"""GPU parity of bf16 problems whose expert weights are packed in MFMA-fragment order
(MOE_DTYPE_BF16_PACKED, weights packed by moe_pack_weights).

The packing is a pure permutation and must be bit-exact against its definition, written
here with numpy. The layer computes the same SwiGLU FFN on the same bf16 values as the
unpacked bf16 path, so every result meets the bf16 tolerances against the fp64 oracle
(on all the small cases of the parity suite, and on sampled rows and a whole expert block
at the workloads' full sizes); stage calls, the gathered gate/up GEMM and repeated calls
are bit-identical to moe_forward.
"""
import numpy as np
import pytest
import torch

import expert_routing_amd as moe
import oracle
from synth import CONFIGS
from gpu_cases import (TOL, cpu_inputs, gpu_inputs, np_, rel_errors, routing_mismatches,
                       run_forward, run_stages)
from test_gpu_parity import SMALL

pytestmark = pytest.mark.gpu

# experts whose remainder under 256-row tiles is 1..64 rows. Their last m-tile is a 64-row
# short tile on packed weights where a GEMM has 2048 tiles or more (the XCDs then split the
# tiles by work): the gate/up GEMM of pk_short64_split (112 n-columns of 2-3 m-tiles per
# expert, two experts ending in 1..64 rows); the smaller cases keep the full last tile.
CASES = dict(SMALL, pk_short64=SMALL["bf16_ragged"].with_(T=1060, h=128, E=4, K=2, inter=192),
             pk_short64_wide=SMALL["bf16_ragged"].with_(T=2100, h=256, E=8, K=2, inter=256),
             pk_short64_split=SMALL["bf16_ragged"].with_(T=2100, h=128, E=8, K=2,
                                                         inter=14336))
BF16_SMALL = [n for n, c in CASES.items() if c.dtype == "bf16"]


def pack_definition(w: np.ndarray) -> np.ndarray:
    """[m][r][c] -> [m][r/32][c/16][64][8]: lane l of block (b, k) holds row 32b + l%32,
    columns 16k + 8(l//32) .. +7."""
    m, r, c = w.shape
    return (w.reshape(m, r // 32, 32, c // 16, 2, 8).transpose(0, 1, 3, 4, 2, 5)
            .reshape(m, r // 32, c // 16, 64, 8))


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy()


@pytest.mark.parametrize("shape", [(1, 32, 16), (3, 64, 48), (2, 96, 128), (5, 160, 208)])
def test_pack_layout_bit_exact(shape):
    g = torch.Generator(device="cuda").manual_seed(sum(shape))
    w = torch.randn(shape, generator=g, device="cuda").to(torch.bfloat16)
    got = moe.pack_weights(w)
    torch.cuda.synchronize()
    ref = pack_definition(_bits(w)).reshape(shape)
    np.testing.assert_array_equal(_bits(got), ref)
    # a 2-D matrix packs as one matrix
    got2 = moe.pack_weights(w[0])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_bits(got2), ref[0])


@pytest.mark.parametrize("name", BF16_SMALL)
def test_packed_layer_parity(name):
    cfg = CASES[name]
    print(f"[case] packed {name} {cfg}", flush=True)
    inp = gpu_inputs(cfg)
    p, b = run_forward(cfg, inp, packed=True)
    inp_c = cpu_inputs(inp)
    rr = oracle.route(K=cfg.K, score=cfg.score, renorm=cfg.renorm, n_groups=cfg.n_groups,
                      topk_groups=cfg.topk_groups, bias=inp_c["bias"], x=inp_c["x"],
                      w_router=inp_c["w_router"])
    ids = np_(b["topk_ids"]).astype(np.int64)
    near, other, _ = routing_mismatches(ids, rr)
    assert other == []
    d = oracle.dispatch(ids, E=cfg.E, n_ep=cfg.n_ep, ep_rank=cfg.ep_rank,
                        capacity_factor=cfg.capacity_factor, pad=cfg.pad, h=cfg.h,
                        dtype_size=cfg.act_bytes)
    np.testing.assert_array_equal(np_(b["offsets"]), d.offsets)
    # the expert FFN on the GPU's own xp against fp64 on the unpacked weights
    xp = b["xp"].cpu()[:d.rows]
    yp_ref = oracle.expert_ffn(xp, d.offsets, inp_c["w13"], inp_c["w2"])
    tmax, tmean = TOL["bf16"]
    mx, mean, zexact = rel_errors(np_(b["yp"])[:d.rows], yp_ref)
    print(f"[ffn] packed {name}: yp max_rel {mx:.3e} mean_rel {mean:.3e}", flush=True)
    assert mx <= tmax and mean <= tmean and zexact, (mx, mean)
    if not near:
        ref = oracle.forward(cfg, inp_c)
        if cfg.n_shared:
            mx, mean, _ = rel_errors(np_(b["y_sh"]), ref["ysh"])
            assert mx <= tmax and mean <= tmean, ("y_sh", mx, mean)
        mx, mean, zexact = rel_errors(np_(b["y"]), ref["y"])
        print(f"[parity] packed {name}: y max_rel {mx:.3e} mean_rel {mean:.3e}", flush=True)
        assert mx <= tmax and mean <= tmean and zexact, (mx, mean)
    # without xp (the gate/up GEMM gathers x): bit-identical
    _, g = run_forward(cfg, inp, gather=True, packed=True)
    assert torch.equal(g["y"], b["y"])
    R = int(b["offsets"][-1].item())
    assert torch.equal(g["yp"][:R], b["yp"][:R])


@pytest.mark.parametrize("name", ["bf16_ragged", "bf16_groups_shared", "bf16_decode",
                                  "bf16_short_last"])
def test_packed_stages_equal_forward_and_repeat(name):
    cfg = SMALL[name]
    inp = gpu_inputs(cfg)
    _, a = run_stages(cfg, inp, packed=True)
    _, f1 = run_forward(cfg, inp, packed=True)
    _, f2 = run_forward(cfg, inp, packed=True)
    for k in ("topk_ids", "counts", "offsets", "dest_row", "y"):
        assert torch.equal(a[k], f1[k]), k
        assert torch.equal(f1[k], f2[k]), k
    if a["y_sh"] is not None:
        assert torch.equal(a["y_sh"], f1["y_sh"])


def _f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


@pytest.mark.parametrize("name", ["mixtral_prefill", "dsv3_ep8", "skew_cap1", "skew_nodrop",
                                  "dsv3_decode"])
def test_packed_full_config(name):
    """The workloads' full sizes: sampled rows of a spread of experts and the whole block
    of the largest one against fp64, and the bench's gathered run bit-identical."""
    cfg = CONFIGS[name]
    print(f"[case] packed full {name}", flush=True)
    inp = gpu_inputs(cfg)
    _, b = run_forward(cfg, inp, packed=True)
    off = np_(b["offsets"]).astype(np.int64)
    El = cfg.E_local
    tmax, tmean = TOL["bf16"]
    rng = np.random.default_rng(1)
    experts = [e for e in range(El) if off[e + 1] > off[e]]
    pick = sorted(set(rng.choice(experts, size=min(8, len(experts)), replace=False).tolist()))
    got, ref = [], []
    for e in pick:
        lo, hi = int(off[e]), int(off[e + 1])
        rows = sorted({lo, hi - 1, (lo + hi) // 2})
        ref.append(oracle.swiglu_ffn(_f64(b["xp"][rows]), _f64(inp["w13"][e]),
                                     _f64(inp["w2"][e])))
        got.append(_f64(b["yp"][rows]))
    mx, mean, _ = rel_errors(np.concatenate(got), np.concatenate(ref))
    print(f"[ffn] packed {name}: sampled rows max_rel {mx:.3e} mean_rel {mean:.3e}", flush=True)
    assert mx <= tmax and mean <= tmean
    big = int(np.argmax(np.diff(off)))
    lo, hi = int(off[big]), int(off[big + 1])
    ref_blk = oracle.swiglu_ffn(_f64(b["xp"][lo:hi]), _f64(inp["w13"][big]),
                                _f64(inp["w2"][big]))
    mx, mean, zexact = rel_errors(_f64(b["yp"][lo:hi]), ref_blk)
    print(f"[ffn] packed {name}: whole block of expert {big} ({hi - lo} rows) max_rel "
          f"{mx:.3e} mean_rel {mean:.3e}", flush=True)
    assert mx <= tmax and mean <= tmean and zexact
    del ref_blk
    y_mat = b["y"].clone()
    del b
    _, g = run_forward(cfg, inp, gather=True, packed=True)
    assert torch.equal(g["y"], y_mat)
