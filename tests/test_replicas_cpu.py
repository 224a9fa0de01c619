"""Host side of the replica map (no GPU): moe_replica_plan equals the oracle's plan
exactly, the sizing call follows the physical-expert layout, and bad arguments are refused."""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import expert_routing_amd as moe
from oracle import replicas as RP


@settings(max_examples=300, deadline=None)
@given(st.lists(st.integers(0, 10 ** 6), min_size=1, max_size=40), st.integers(0, 24),
       st.sampled_from([1, 2, 4, 8]))
def test_plan_matches_oracle(load, R, n_ep):
    E = len(load)
    if (E + R) % n_ep:
        R += n_ep - (E + R) % n_ep
    got = moe.replica_plan(E, R, n_ep, load)
    ref = RP.plan(load, R, n_ep)
    for k in ("counts", "rep_start", "rep_list", "phys_expert", "phys_replica"):
        np.testing.assert_array_equal(got[k], getattr(ref, k), err_msg=k)


def test_plan_at_the_pages_example():
    # 256 logical + 32 redundant = 288 physical experts over 8 ranks (36 each), skewed loads
    rng = np.random.default_rng(0)
    load = rng.zipf(1.5, size=256).clip(max=10 ** 6)
    got = moe.replica_plan(256, 32, 8, load)
    ref = RP.plan(load, 32, 8)
    np.testing.assert_array_equal(got["phys_expert"], ref.phys_expert)
    assert got["counts"].sum() == 288 and len(got["rep_list"]) == 288


@pytest.mark.parametrize("args", [(0, 0, 1), (513, 0, 1), (8, -1, 1), (8, 1, 2), (8, 0, 0)])
def test_plan_refuses_bad_arguments(args):
    E, R, N = args
    with pytest.raises(moe.MoeError):
        moe.replica_plan(E, R, N, [1] * max(E, 1))


def test_replicated_sizes():
    p = moe.Problem(T=100, h=64, E=16, K=3, inter=64, n_ep=4, capacity_factor=1.0)
    rows, ws = moe.replicated_sizes(p, 24)           # 6 physical experts per rank
    cap = RP.capacity_physical(1.0, 100, 3, 24)
    assert rows == min(100 * 3, 6 * cap) and ws > 0
    p0 = moe.Problem(T=100, h=64, E=16, K=3, inter=64, n_ep=4)
    assert moe.replicated_sizes(p0, 24)[0] == 100 * 3
    with pytest.raises(moe.MoeError):
        moe.replicated_sizes(p0, 15)                  # fewer physical than logical
    with pytest.raises(moe.MoeError):
        moe.replicated_sizes(p0, 18)                  # not a multiple of the ranks
