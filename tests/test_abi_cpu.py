"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every
entry point include/moe.h declares, validates problems before any launch, and sizes
capacity / rows exactly as the oracle's definitions do."""
import os
import re

import pytest
from hypothesis import given, settings, strategies as st

import oracle
import expert_routing_amd as moe
from synth import CONFIGS

HDR = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "moe.h")


def declared_symbols():
    txt = open(HDR).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", txt)))


def test_every_declared_symbol_is_exported():
    syms = declared_symbols()
    assert len(syms) >= 10
    for s in syms:
        assert hasattr(moe._lib, s), s
    assert sorted(moe.EXPORTED) == syms


def test_status_strings():
    assert moe.status_string(0) == "ok"
    assert "invalid" in moe.status_string(-1)
    assert "workspace" in moe.status_string(-3)


@pytest.mark.parametrize("name", list(CONFIGS))
def test_configs_are_valid(name):
    cfg = CONFIGS[name]
    p = moe.problem_from_config(cfg)
    assert moe.check_problem(p) == 0
    cap = oracle.capacity(cfg.capacity_factor, cfg.T, cfg.K, cfg.E)
    assert moe.capacity(p) == (-1 if cap is None else cap)
    assert moe.max_rows(p) == oracle.max_rows(cfg.T, cfg.K, cfg.E, cfg.n_ep, cap, cfg.pad)
    assert moe.workspace_bytes(p) > 0


@settings(max_examples=300, deadline=None)
@given(st.floats(0.01, 8.0, allow_nan=False), st.integers(0, 100000), st.integers(1, 16),
       st.sampled_from([1, 2, 8, 16, 64, 256, 512]))
def test_capacity_exact_matches_oracle(cf, T, K, E):
    K = min(K, E)
    p = moe.Problem(T=T, h=64, E=E, K=K, capacity_factor=cf, inter=64)
    assert moe.capacity(p) == oracle.capacity(cf, T, K, E)


@pytest.mark.parametrize("pad", [False, True])
def test_max_rows(pad):
    for (T, K, E, N, cf) in [(64, 2, 8, 1, 1.25), (100, 4, 16, 4, 0.5), (7, 3, 6, 2, 2.0),
                             (32, 8, 256, 1, 0.0), (512, 8, 256, 64, 1.0)]:
        if pad and cf <= 0:
            continue
        p = moe.Problem(T=T, h=64, E=E, K=K, capacity_factor=cf, pad=pad, n_ep=N, inter=64)
        cap = oracle.capacity(cf, T, K, E)
        assert moe.max_rows(p) == oracle.max_rows(T, K, E, N, cap, pad)


INVALID = [
    dict(T=-1), dict(h=0), dict(E=0), dict(E=513, K=2), dict(K=0), dict(K=9, E=8),
    dict(K=17, E=64), dict(n_ep=3), dict(ep_rank=1), dict(n_groups=3),
    dict(n_groups=4, topk_groups=0), dict(n_groups=4, topk_groups=5),
    dict(n_groups=8, topk_groups=1, K=2),                 # 1 group of 1 expert < K
    dict(pad=True), dict(n_shared=2), dict(n_shared=1, shared_inter=0),
    dict(n_shared=1, shared_inter=64, n_ep=2, T=33),
]


@pytest.mark.parametrize("kw", INVALID)
def test_invalid_problems(kw):
    base = dict(T=32, h=64, E=8, K=2, inter=64)
    base.update(kw)
    p = moe.Problem(**base)
    assert moe.check_problem(p) == -1
    # entry points refuse before touching the device (no GPU here)
    assert moe._route(moe.ctypes.byref(p), None, None, None, None, None, None, 0, None) == -1


@pytest.mark.parametrize("kw", [dict(h=96), dict(inter=96), dict(n_shared=1, shared_inter=32)])
def test_unsupported_bf16_shapes(kw):
    base = dict(T=32, h=64, E=8, K=2, inter=64)
    base.update(kw)
    assert moe.check_problem(moe.Problem(**base)) == -2
    base["dtype"] = "f32"
    assert moe.check_problem(moe.Problem(**base)) == 0


def test_bf16_operand_offset_limits():
    # the GEMMs' 32-bit byte offsets: tokens x hidden and 2*inter x hidden must fit
    ok = dict(T=262144, h=7168, E=8, K=2, inter=2048)          # x = 3.5 GiB
    assert moe.check_problem(moe.Problem(**ok)) == 0
    assert moe.check_problem(moe.Problem(**dict(ok, T=300000))) == -2
    assert moe.check_problem(moe.Problem(**dict(ok, T=64, inter=1 << 17))) == 0   # 3.8 GB
    assert moe.check_problem(moe.Problem(**dict(ok, T=64, inter=3 << 16))) == -2  # 5.6 GB
    assert moe.check_problem(moe.Problem(**dict(ok, T=300000, dtype="f32"))) == 0


def test_null_and_workspace_errors_before_launch():
    p = moe.Problem(T=32, h=64, E=8, K=2, inter=64)
    b = moe.ctypes.byref(p)
    fake = 0x1000  # never dereferenced: validation fails first
    assert moe._route(b, None, fake, None, fake, fake, fake, 1 << 30, None) == -1
    assert moe._route(b, fake, fake, None, fake, fake, None, 0, None) == -3
    assert moe._route(b, fake, fake, None, fake, fake, fake + 8, 1 << 30, None) == -3
    assert moe._route(b, fake, fake, None, fake, fake, fake, 16, None) == -3
    # dispatch: x and xp must both be given or both be NULL
    assert moe._dispatch(b, fake, fake, fake, fake, fake, fake, None, fake, None,
                         fake, 1 << 30, None) == -1
    # send matrix needs T % n_ep == 0
    p2 = moe.Problem(T=33, h=64, E=8, K=2, inter=64, n_ep=2)
    assert moe._dispatch(moe.ctypes.byref(p2), None, fake, fake, fake, fake, fake, fake, fake,
                         None, fake, 1 << 30, None) == -1
    # ffn without shared expert must not get shared pointers
    assert moe._expert_ffn(b, fake, None, fake, fake, fake, fake, fake, fake, fake, None, fake,
                           1 << 30, None) == -1
    # ffn without xp needs row_src and x (the gathered gate/up rows)
    assert moe._expert_ffn(b, None, None, fake, fake, fake, fake, None, None, fake, None, fake,
                           1 << 30, None) == -1
    assert moe._expert_ffn(b, None, fake, fake, fake, fake, None, None, None, fake, None, fake,
                           1 << 30, None) == -1
    assert moe._combine(b, fake, None, fake, None, fake, None) == -1
    assert moe._forward(b, None, fake, 1 << 30, None) == -1
    # layout statistics: ids required; tokens_to needs T % n_ep == 0; workspace checked
    assert moe._layout_stats(b, None, fake, fake, fake, fake, fake, 1 << 30, None) == -1
    assert moe._layout_stats(moe.ctypes.byref(p2), fake, fake, None, None, None, fake, 1 << 30,
                             None) == -1
    assert moe._layout_stats(b, fake, fake, fake, fake, fake, fake, 16, None) == -3


def test_empty_batch_is_a_no_op():
    p = moe.Problem(T=0, h=64, E=8, K=2, inter=64)
    b = moe.ctypes.byref(p)
    assert moe.max_rows(p) == 0
    assert moe._route(b, None, None, None, None, None, None, 0, None) == 0
    assert moe._select(b, None, None, None, None, None) == 0
    assert moe._combine(b, None, None, None, None, None, None) == 0


def test_noalloc_refuses_problems_beyond_its_scratch():
    # the Mixtral-shaped layer needs ~288 MiB of workspace: refused before any launch
    p = moe.problem_from_config(CONFIGS["mixtral_prefill"])
    assert moe.workspace_bytes(p) > moe.NOALLOC_SCRATCH_BYTES
    assert moe._forward_noalloc(moe.ctypes.byref(p), None, None) == -3
    # invalid problems are reported as such first
    bad = moe.Problem(T=32, h=64, E=8, K=9, inter=64)
    assert moe._forward_noalloc(moe.ctypes.byref(bad), None, None) == -1


def test_pack_weights_argument_checks():
    fake, other = 0x10000, 0x20000000   # never dereferenced: validation fails first
    pk = moe._pack_weights
    assert pk(0, 32, 16, None, None, None) == 0                 # nothing to pack
    assert pk(-1, 32, 16, fake, other, None) == -1
    assert pk(1, 48, 16, fake, other, None) == -1               # rows % 32
    assert pk(1, 32, 24, fake, other, None) == -1               # cols % 16
    assert pk(1, 32, 16, None, other, None) == -1
    assert pk(1, 32, 16, fake + 8, other, None) == -1           # 16-byte alignment
    assert pk(2, 64, 64, fake, fake + 4096, None) == -1         # overlapping
    assert pk(1, 32, 16, fake, fake, None) == -1                # in place


def test_packed_dtype_is_a_bf16_problem():
    ok = dict(T=64, h=128, E=8, K=2, inter=128)
    assert moe.check_problem(moe.Problem(**ok, dtype="bf16_packed")) == 0
    assert moe.check_problem(moe.Problem(**dict(ok, h=96), dtype="bf16_packed")) == -2
    p = moe.Problem(**ok, dtype="bf16_packed")
    assert p.torch_dtype == moe.torch.bfloat16
    assert moe.workspace_bytes(p) == moe.workspace_bytes(moe.Problem(**ok))
