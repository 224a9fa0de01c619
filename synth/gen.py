"""Seeded input generators.

Every tensor has its own seed, derived from the workload seed and the tensor's name
(and, for expert weights, the global expert id), so one expert's weights can be
regenerated alone. Values come from torch's generator on the requested device:
MT19937 on the CPU, Philox on a GPU. The two devices therefore give different (but
equally distributed) draws; a parity check always hands the oracle the very tensors
the GPU path consumed, copied to the host.

Distributions (the second argument of N(., .) is a variance):
  x ~ N(0, 1);  W_r ~ N(0, 1/h) in fp32, stored [E, h];  expert weights ~ N(0, 1/fan_in);
  gauss bias ~ N(0, bias_var) in fp32;  zipf bias b_e = -s * ln(rank_e) with rank_e a
  seeded permutation of 1..E;  uniform keys ~ U(0, 1) in fp32.
Activations and expert weights are rounded to the workload dtype by torch's cast
(round to nearest even for bf16).
"""
from __future__ import annotations

import hashlib
import math

import torch

from .configs import MoEConfig

_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


def sub_seed(seed: int, *names) -> int:
    """A 63-bit seed derived from the workload seed and a tensor's name parts."""
    h = hashlib.blake2b(repr((int(seed),) + tuple(names)).encode(), digest_size=8)
    return int.from_bytes(h.digest(), "little") & ((1 << 63) - 1)


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(seed)
    return g


def _normal(shape, std: float, seed: int, device, dtype) -> torch.Tensor:
    g = _gen(device, seed)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def act_dtype(cfg: MoEConfig) -> torch.dtype:
    return _DTYPES[cfg.dtype]


def make_expert_weights(cfg: MoEConfig, e: int, device="cpu", shared: bool = False):
    """(w13, w2) of one expert: w13 is [2I, h] (gate rows, then up rows), w2 is [h, I].

    `e` is the global expert id (or the shared expert's index when shared=True).
    """
    dt = act_dtype(cfg)
    inter = cfg.shared_inter if shared else cfg.inter
    tag = "shared" if shared else "routed"
    w13 = _normal((2 * inter, cfg.h), 1.0 / math.sqrt(cfg.h),
                  sub_seed(cfg.seed, tag, "w13", e), device, dt)
    w2 = _normal((cfg.h, inter), 1.0 / math.sqrt(inter),
                 sub_seed(cfg.seed, tag, "w2", e), device, dt)
    return w13, w2


def make_bias(cfg: MoEConfig, device="cpu"):
    if cfg.bias == "none":
        return None
    if cfg.bias == "gauss":
        return _normal((cfg.E,), math.sqrt(cfg.bias_var), sub_seed(cfg.seed, "bias"),
                       device, torch.float32)
    if cfg.bias == "zipf":
        g = _gen("cpu", sub_seed(cfg.seed, "zipf_rank"))
        rank = torch.randperm(cfg.E, generator=g).to(torch.float64) + 1.0
        return (-cfg.zipf_s * torch.log(rank)).to(torch.float32).to(device)
    raise ValueError(cfg.bias)


def make_inputs(cfg: MoEConfig, device="cpu", with_weights: bool = True,
                T: int | None = None) -> dict:
    """All inputs of one layer call. `T` overrides the token count (token rows are
    drawn from the same stream, so a smaller T gives a prefix of the full x)."""
    T = cfg.T if T is None else T
    dt = act_dtype(cfg)
    out = {"cfg": cfg, "T": T}
    if cfg.keys == "uniform":
        g = _gen(device, sub_seed(cfg.seed, "keys"))
        out["keys"] = torch.rand((cfg.T, cfg.E), generator=g, device=device)[:T].contiguous()
        out["x"] = None
        out["w_router"] = None
    else:
        out["x"] = _normal((cfg.T, cfg.h), 1.0, sub_seed(cfg.seed, "x"), device, dt)[:T].contiguous()
        out["w_router"] = _normal((cfg.E, cfg.h), 1.0 / math.sqrt(cfg.h),
                                  sub_seed(cfg.seed, "w_router"), device, torch.float32)
    out["bias"] = make_bias(cfg, device)
    if with_weights and cfg.inter > 0:
        El, e0 = cfg.E_local, cfg.ep_rank * cfg.E_local
        w13 = torch.empty((El, 2 * cfg.inter, cfg.h), dtype=dt, device=device)
        w2 = torch.empty((El, cfg.h, cfg.inter), dtype=dt, device=device)
        for el in range(El):
            a, b = make_expert_weights(cfg, e0 + el, device)
            w13[el].copy_(a)
            w2[el].copy_(b)
            del a, b
        out["w13"], out["w2"] = w13, w2
        if cfg.n_shared:
            out["w13_sh"], out["w2_sh"] = make_expert_weights(cfg, 0, device, shared=True)
        else:
            out["w13_sh"] = out["w2_sh"] = None
    return out
