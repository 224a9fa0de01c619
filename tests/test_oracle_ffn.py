"""Pins for the oracle's expert FFN, combine and full forward (CPU only).

Ground truth: torch's float64 CPU ops (F.linear with the [out, in] weight convention,
F.silu) for the dense SwiGLU special case, and reductions of the whole layer to a dense
FFN (one expert; identical experts), plus brute-force combine sums."""
import numpy as np
import torch
import torch.nn.functional as F

import oracle
from oracle.dispatch import permute
from synth import CONFIGS, make_inputs


def dense_swiglu_torch(x, w13, w2):
    x, w13, w2 = (torch.as_tensor(np.asarray(a, np.float64)) for a in (x, w13, w2))
    inter = w13.shape[0] // 2
    g = F.linear(x, w13[:inter])
    u = F.linear(x, w13[inter:])
    return F.linear(F.silu(g) * u, w2).numpy()


def test_swiglu_matches_torch_library():
    rng = np.random.default_rng(0)
    x = rng.normal(size=(7, 12))
    w13 = rng.normal(size=(2 * 5, 12))
    w2 = rng.normal(size=(12, 5))
    np.testing.assert_allclose(oracle.swiglu_ffn(x, w13, w2), dense_swiglu_torch(x, w13, w2),
                               rtol=1e-12, atol=1e-12)


def test_gate_and_up_are_not_swapped():
    # silu(g)*u is not symmetric in (g, u): swapping the halves must change the result
    rng = np.random.default_rng(1)
    x = rng.normal(size=(3, 4))
    w13 = rng.normal(size=(6, 4))
    w2 = rng.normal(size=(4, 3))
    swapped = np.concatenate([w13[3:], w13[:3]])
    assert not np.allclose(oracle.swiglu_ffn(x, w13, w2), oracle.swiglu_ffn(x, swapped, w2))


def test_silu_zero():
    w13 = np.zeros((4, 3))
    w2 = np.ones((3, 2))
    assert (oracle.swiglu_ffn(np.ones((2, 3)), w13, w2) == 0).all()


def test_single_expert_layer_is_dense_ffn():
    """K = E = 1 with no capacity: every token goes to the one expert with weight 1."""
    cfg = CONFIGS["tiny_f32"].with_(E=1, K=1, capacity_factor=0.0, T=16, h=32, inter=24)
    inp = make_inputs(cfg)
    out = oracle.forward(cfg, inp)
    assert (out["route"].weights == 1.0).all()
    ref = dense_swiglu_torch(inp["x"].numpy(), inp["w13"][0].numpy(), inp["w2"][0].numpy())
    np.testing.assert_allclose(out["y"], ref, rtol=1e-12, atol=1e-12)


def test_identical_experts_give_dense_ffn():
    """All experts share the same weights and the weights sum to 1: y = FFN(x)."""
    cfg = CONFIGS["tiny_f32"].with_(capacity_factor=0.0, T=24, h=32, inter=16)
    inp = make_inputs(cfg)
    inp["w13"][:] = inp["w13"][0]
    inp["w2"][:] = inp["w2"][0]
    out = oracle.forward(cfg, inp)
    ref = dense_swiglu_torch(inp["x"].numpy(), inp["w13"][0].numpy(), inp["w2"][0].numpy())
    np.testing.assert_allclose(out["y"], ref, rtol=1e-11, atol=1e-12)


def test_combine_brute_force_and_drops():
    cfg = CONFIGS["tiny_f32"].with_(capacity_factor=0.5, T=40, h=16, inter=8)
    inp = make_inputs(cfg)
    out = oracle.forward(cfg, inp)
    d, rr = out["dispatch"], out["route"]
    x = inp["x"].numpy().astype(np.float64)
    assert d.n_dropped > 0
    for t in range(cfg.T):
        acc = np.zeros(cfg.h)
        for k in range(cfg.K):
            if d.kept[t, k]:
                e = rr.ids[t, k]
                acc += rr.weights[t, k] * dense_swiglu_torch(
                    x[t:t + 1], inp["w13"][e].numpy(), inp["w2"][e].numpy())[0]
        np.testing.assert_allclose(out["y"][t], acc, rtol=1e-11, atol=1e-13)
        if not d.kept[t].any():
            assert (out["y"][t] == 0).all()


def test_shared_expert_on_local_block_only():
    cfg = CONFIGS["dsv3_ep8"].with_(T=32, h=16, E=16, K=4, n_groups=4, topk_groups=2,
                                    inter=8, shared_inter=8, n_ep=4, ep_rank=1, dtype="f32")
    inp = make_inputs(cfg)
    out = oracle.forward(cfg, inp)
    x = inp["x"].numpy().astype(np.float64)
    t0, t1 = 8, 16
    sh = dense_swiglu_torch(x[t0:t1], inp["w13_sh"].numpy(), inp["w2_sh"].numpy())
    routed = oracle.combine(out["yp"], out["dispatch"].dest_row, out["route"].weights)
    np.testing.assert_allclose(out["y"][t0:t1], routed[t0:t1] + sh, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(out["y"][:t0], routed[:t0])
    np.testing.assert_array_equal(out["y"][t1:], routed[t1:])
    # only local experts (4..7) own rows
    d = out["dispatch"]
    live = d.row_src[d.row_src >= 0]
    e_of = out["route"].ids.reshape(-1)[live]
    assert ((e_of >= 4) & (e_of < 8)).all()


def test_padded_layout_gives_same_output():
    cfg = CONFIGS["tiny_f32"].with_(capacity_factor=1.0, T=32, h=16, inter=8)
    inp = make_inputs(cfg)
    a = oracle.forward(cfg, inp)
    b = oracle.forward(cfg.with_(pad=True), inp)
    np.testing.assert_array_equal(a["y"], b["y"])
    xp = permute(inp["x"].numpy(), b["dispatch"], cfg.K)
    assert xp.shape[0] == cfg.E * b["dispatch"].cap
