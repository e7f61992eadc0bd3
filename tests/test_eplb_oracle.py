"""Pins of the EPLB oracle (``oracle/eplb_oracle.py``) against what the pages
and the mathematics fix, independent of the oracle's own code paths.

"Serving MoE models with expert parallelism on 8xH200" (reviosa), section
"Routing imbalance": the imbalance factor is the busiest GPU's token count
over the mean; hot experts get redundant copies on less-loaded GPUs; hot and
cold experts share GPUs.
"""
import itertools
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import eplb_oracle as eo
from oracle import moe_oracle as mo

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "eplb_hand_example.json")


def brute_force_min_max_per_copy(load, G, R):
    """min over every copy assignment (1..G copies per expert, E+R in all)
    of the largest load per copy, exactly."""
    E = len(load)
    best = None
    for reps in itertools.product(range(1, G + 1), repeat=E):
        if sum(reps) != E + R:
            continue
        m = max(Fraction(c, r) for c, r in zip(load, reps))
        best = m if best is None or m < best else best
    return best


@pytest.mark.parametrize("seed", range(12))
def test_replication_minimises_the_largest_load_per_copy(seed):
    # greedy copying of the largest load-per-copy is optimal for that
    # objective; check against enumeration of all copy vectors
    rng = np.random.default_rng(seed)
    E = int(rng.integers(2, 5))
    G = int(rng.integers(2, 4))
    R = int(rng.integers(0, E * (G - 1) + 1))
    R -= (E + R) % G
    if R < 0:
        R += G
    load = [int(v) for v in rng.integers(0, 50, size=E)]
    rep, _, _, _ = eo.plan(load, G, R)
    assert int(rep.sum()) == E + R and rep.min() >= 1 and rep.max() <= G
    got = max(Fraction(c, int(r)) for c, r in zip(load, rep))
    assert got == brute_force_min_max_per_copy(load, G, R)


def test_hand_worked_example():
    # worked by hand in tests/golden/eplb_hand_example.json
    ex = json.load(open(GOLDEN))
    rep, p2l, l2p, rank_load = eo.plan(ex["load"], ex["G"], ex["R"])
    assert rep.tolist() == ex["replicas"]
    assert p2l.tolist() == ex["phys_to_log"]
    assert l2p.tolist() == ex["log_to_phys"]
    assert rank_load.tolist() == ex["rank_load"]
    rank_of = eo.contiguous_rank_of_expert(len(ex["load"]), ex["G"])
    before = np.bincount(rank_of, weights=ex["load"], minlength=ex["G"])
    assert eo.imbalance_factor(before) == pytest.approx(ex["imbalance_contiguous"], rel=1e-15)
    assert eo.imbalance_factor(rank_load) == ex["imbalance_plan"]


def test_uniform_load_is_balanced():
    rep, p2l, _, rank_load = eo.plan([7] * 32, 8, 0)
    assert rep.tolist() == [1] * 32
    assert sorted(p2l.tolist()) == list(range(32))
    assert rank_load.tolist() == [28.0] * 8
    assert eo.imbalance_factor(rank_load) == 1.0


def test_single_hot_expert_spreads_over_every_rank():
    # one expert with 8x the total of the rest: with G - 1 spare slots it
    # gets a copy on every rank, and the rest fill the ranks evenly
    G, E = 4, 12
    load = [800] + [10] * (E - 1)
    R = G  # P = 16, 4 slots per rank
    rep, p2l, l2p, rank_load = eo.plan(load, G, R)
    assert rep[0] == G
    ranks_of_hot = sorted(int(p) // 4 for p in l2p[0] if p >= 0)
    assert ranks_of_hot == [0, 1, 2, 3]
    # 800/4 = 200 per copy; the 11 cold experts plus one extra copy of
    # expert 1 (10/2 = 5 each) share the remaining 12 slots
    assert rep[1] == 2 and rep[2:].tolist() == [1] * (E - 2)
    assert sum(rank_load) == pytest.approx(sum(load))
    assert eo.imbalance_factor(rank_load) == pytest.approx(
        (200 + 30) / (sum(load) / G))


def zipf_loads(E, s, total, seed):
    rng = np.random.default_rng(seed)
    p = (np.arange(E) + 1.0) ** (-s)
    return rng.multinomial(total, p / p.sum())


@pytest.mark.parametrize("R", [0, 8, 16, 32])
def test_plan_invariants_on_skewed_loads(R):
    E, G = 256, 8
    load = zipf_loads(E, 1.2, 131072, seed=R)
    rep, p2l, l2p, rank_load = eo.plan(load, G, R)
    P, S = E + R, (E + R) // G
    assert int(rep.sum()) == P
    # every slot holds an expert; expert e appears rep[e] times
    assert np.bincount(p2l, minlength=E).tolist() == rep.tolist()
    for e in range(E):
        ps = [int(p) for p in l2p[e] if p >= 0]
        assert len(ps) == rep[e] and ps == sorted(ps)
        assert all(p2l[p] == e for p in ps)
        assert len({p // S for p in ps}) == len(ps), "copies of one expert share a rank"
        assert (l2p[e, len(ps):] == -1).all()
    # physical ids in a rank are in increasing expert order
    for g in range(G):
        blk = p2l[g * S:(g + 1) * S]
        assert (np.diff(blk) >= 0).all()
    exact = eo.predicted_rank_loads(load, rep, p2l, G)
    assert np.allclose(rank_load, exact, rtol=1e-12, atol=0)
    assert exact.sum() == pytest.approx(load.sum(), rel=1e-12)
    before = np.bincount(eo.contiguous_rank_of_expert(E, G), weights=load, minlength=G)
    assert eo.imbalance_factor(rank_load) < eo.imbalance_factor(before)
    # the pages' threshold: a skew this strong is above 1.3 before the plan
    assert eo.imbalance_factor(before) > 1.3


def test_more_copies_never_raise_the_largest_copy():
    load = zipf_loads(64, 1.1, 20000, seed=3)
    prev = None
    for R in (0, 8, 16, 24, 32):
        rep, _, _, _ = eo.plan(load, 8, R)
        m = max(Fraction(int(c), int(r)) for c, r in zip(load, rep))
        assert prev is None or m <= prev
        prev = m


def test_remap_sends_slot_to_copy_t_mod_replicas():
    rng = np.random.default_rng(7)
    T, k, E, G, R = 50, 3, 8, 4, 4
    load = rng.integers(0, 100, size=E)
    rep, p2l, l2p, _ = eo.plan(load, G, R)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    idx[3, 1] = -1
    idx[4, 2] = E + 5
    phys = eo.remap(idx, rep, l2p)
    assert phys[3, 1] == -1 and phys[4, 2] == -1
    # brute force: copy j of expert e receives exactly the slots of the tokens
    # t with t % rep[e] == j
    for e in range(E):
        for j in range(int(rep[e])):
            want = sorted((t, i) for t in range(T) for i in range(k)
                          if idx[t, i] == e and t % rep[e] == j)
            got = sorted((t, i) for t in range(T) for i in range(k) if phys[t, i] == l2p[e, j])
            assert got == want
    ok = (idx >= 0) & (idx < E)
    assert (p2l[phys[ok]] == idx[ok]).all()


def test_ranks_with_copies_sum_to_the_whole_layer():
    # the plan changes where slots run, never what the layer computes: with
    # physical copies of the weights, the G ranks' partial outputs add up to
    # the single-device layer
    rng = np.random.default_rng(11)
    T, d, E, k, F, G, R = 24, 16, 6, 2, 8, 3, 3
    x = rng.standard_normal((T, d)).astype(np.float32)
    L = (rng.standard_normal((T, E)) + np.array([2.0, 1.0, 0, 0, 0, 0])).astype(np.float32)
    wg = rng.standard_normal((E, F, d)).astype(np.float32)
    wu = rng.standard_normal((E, F, d)).astype(np.float32)
    wd = rng.standard_normal((E, d, F)).astype(np.float32)
    full = mo.moe_layer_forward(x, L, k, wg, wu, wd, act_fmt="f32", weight_fmt="f32")
    counts = np.bincount(full["topk_idx"].reshape(-1), minlength=E)
    rep, p2l, l2p, _ = eo.plan(counts, G, R)
    phys = eo.remap(full["topk_idx"], rep, l2p)
    S = (E + R) // G
    acc = np.zeros((T, d))
    for g in range(G):
        blk = p2l[g * S:(g + 1) * S]
        part = mo.routed_layer_forward(x, phys, full["topk_w"], wg[blk], wu[blk], wd[blk],
                                       act_fmt="f32", weight_fmt="f32", e0=g * S, E_l=S)
        acc += part["out"]
    np.testing.assert_allclose(acc, full["out"], rtol=1e-12, atol=1e-12)
    # the realised per-rank slot counts
    rank_of_phys = np.arange(E + R) // S
    per_rank = eo.rank_slot_counts(phys, rank_of_phys, G)
    assert per_rank.sum() == T * k


def test_invalid_arguments():
    with pytest.raises(ValueError):
        eo.plan([1, 2, 3], 2, 0)      # P = 3 not divisible by 2
    with pytest.raises(ValueError):
        eo.plan([1, 2], 2, 4)         # more copies than ranks per expert
    with pytest.raises(ValueError):
        eo.plan([1, -2], 2, 0)
