"""The library's EPLB placement plan (host code behind moe_eplb_plan) against
the oracle, bit for bit, and its argument checks.  Host only: no GPU."""
import os

import numpy as np
import pytest

from mixture_experts_layer_15_amd import binding as B
from oracle import eplb_oracle as eo


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from mixture_experts_layer_15_amd import build
        build.build()
    return B.load_library()


def same_plan(load, G, R):
    got = B.moe_eplb_plan(load, G, R)
    want = eo.plan(load, G, R)
    for g, w, name in zip(got, want, ("replicas", "phys_to_log", "log_to_phys", "rank_load")):
        assert g.shape == w.shape, name
        assert np.array_equal(g, w), name  # float64 rank loads too: same sums in the same order


def zipf_counts(E, s, total, seed):
    rng = np.random.default_rng(seed)
    p = (np.arange(E) + 1.0) ** (-s)
    return rng.multinomial(total, p / p.sum())


@pytest.mark.parametrize("R", [0, 8, 16, 32, 64])
def test_plan_matches_oracle_deepseek_shape(lib, R):
    # 256 routed experts on 8 ranks (the pages' DeepSeek-V3 EP layout), Zipf-skewed counts
    same_plan(zipf_counts(256, 1.2, 16384 * 8, seed=R), 8, R)


@pytest.mark.parametrize("seed", range(40))
def test_plan_matches_oracle_random(lib, seed):
    rng = np.random.default_rng(100 + seed)
    E = int(rng.integers(1, 40))
    G = int(rng.integers(1, 9))
    R = int(rng.integers(0, E * (G - 1) + 1)) if G > 1 else 0
    R -= (E + R) % G
    if R < 0:
        R += G
    if R > E * (G - 1) or E + R > 512:
        pytest.skip("no valid R for this draw")
    kind = seed % 4
    if kind == 0:
        load = rng.integers(0, 1000, size=E)
    elif kind == 1:
        load = rng.integers(0, 4, size=E) * 10      # many equal loads: tie rules
    elif kind == 2:
        load = np.zeros(E, dtype=np.int64)          # all idle
    else:
        load = rng.integers(0, 2**40, size=E)       # near the limit
    same_plan(load, G, R)


def test_plan_every_expert_copied_to_every_rank(lib):
    # R = E (G - 1): every expert on every rank
    same_plan([5, 1, 3], 4, 9)
    rep, p2l, l2p, _ = B.moe_eplb_plan([5, 1, 3], 4, 9)
    assert rep.tolist() == [4, 4, 4]
    assert sorted(p2l.tolist()) == [0] * 4 + [1] * 4 + [2] * 4


def test_plan_small_edge_cases(lib):
    # one dominant expert, equal pairs, all load on the last expert.  (The
    # rule for a copy that finds only ranks already holding its expert is
    # never reached here: a random search over small plans found no
    # such case, since an expert's copies are placed one after another.)
    for load, G, R in (([100, 1, 1, 1, 1, 1], 3, 3), ([9, 9, 1, 1], 2, 2), ([0, 0, 0, 7], 4, 4)):
        same_plan(load, G, R)


@pytest.mark.parametrize("args", [
    (np.array([1, 2, 3]), 2, 0),      # P not divisible by G
    (np.array([1, 2]), 2, 3),         # R > E (G - 1)
    (np.array([1, 2]), 0, 0),         # G = 0
    (np.array([1, 2]), 2, -2),        # R < 0
    (np.array([1, -1]), 1, 0),        # negative load
    (np.array([2**40, 1]), 1, 0),     # load at 2^40
])
def test_plan_rejects_invalid(lib, args):
    with pytest.raises(B.MoEError) as ei:
        B.moe_eplb_plan(*args)
    assert ei.value.status == B.MOE_ERR_INVALID_ARGUMENT


def test_plan_too_many_slots_unsupported(lib):
    with pytest.raises(B.MoEError) as ei:
        B.moe_eplb_plan(np.ones(512), 2, 2)
    assert ei.value.status == B.MOE_ERR_UNSUPPORTED


def test_remap_argument_checks(lib):
    # host checks only (no kernel is launched for any of these)
    for T, k, E, G in ((-1, 2, 4, 2), (4, 0, 4, 2), (4, 2, 0, 2), (4, 2, 4, 0)):
        assert lib.moe_eplb_remap(T, k, E, G, 16, 16, 16, 16, None) == B.MOE_ERR_INVALID_ARGUMENT
    assert lib.moe_eplb_remap(4, 2, 4, 2, None, 16, 16, 16, None) == B.MOE_ERR_INVALID_ARGUMENT
    assert lib.moe_eplb_remap(1 << 30, 4, 4, 2, 16, 16, 16, 16, None) == B.MOE_ERR_UNSUPPORTED
    assert lib.moe_eplb_remap(0, 2, 4, 2, 16, 16, 16, 16, None) == B.MOE_OK
