"""Pins of the CPU oracle to things other than itself.

Each test checks the oracle against a library routine, a closed form, an
invariant the method fixes, brute force on tiny inputs, or a figure printed on
the pages (``tests/golden/pages_figures.json``).  They are chosen so that a
plausible slip in the oracle (a dropped term, a flipped sign, a wrong index, a
transposed operand) fails at least one of them.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as Fnn

from oracle import moe_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_figures.json")


def _f32_problem(rng, T, d, E, k, F, E_l=None, e0=0, bias=False):
    """Small float32 problem in the storage layout the oracle takes."""
    E_l = E - e0 if E_l is None else E_l
    x = rng.standard_normal((T, d)).astype(np.float32)
    w_r = (rng.standard_normal((d, E)) / np.sqrt(d)).astype(np.float32)
    b = (rng.standard_normal(E)).astype(np.float32) if bias else None
    wg = (rng.standard_normal((E_l, F, d)) / np.sqrt(d)).astype(np.float32)
    wu = (rng.standard_normal((E_l, F, d)) / np.sqrt(d)).astype(np.float32)
    wd = (rng.standard_normal((E_l, d, F)) / np.sqrt(F)).astype(np.float32)
    L = orc.router_logits(x.astype(np.float64), w_r.astype(np.float64), b).astype(np.float32)
    return x, L, wg, wu, wd


# ---------------------------------------------------------------- decoding

def test_bf16_decode_all_patterns_match_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = orc.bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_e4m3fn_table_matches_torch_and_format_facts():
    tab = orc.e4m3fn_table()
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(tab), nan)
    assert np.array_equal(tab[~nan], ref[~nan])
    # OCP E4M3FN: NaN only at S.1111.111, no infinities, max 448, min subnormal 2^-9
    assert list(np.nonzero(np.isnan(tab))[0]) == [0x7F, 0xFF]
    assert not np.isinf(tab).any()
    assert np.nanmax(tab) == 448.0 and np.nanmin(tab) == -448.0
    assert tab[0x01] == 2.0 ** -9 and tab[0x38] == 1.0
    # every finite E4M3FN value is exactly a bfloat16 (3 mantissa bits < 7)
    fin = tab[~np.isnan(tab)]
    as_bf16 = torch.from_numpy(fin).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(as_bf16, fin)


def test_dequant_block_layout_is_kron_of_scales():
    # non-square block grid (2 x 3 blocks) with distinct scales: a transposed
    # or swapped block index cannot pass
    rng = np.random.default_rng(0)
    s = rng.uniform(0.5, 3.0, size=(2, 3)).astype(np.float32)
    ones = np.full((256, 384), 0x38, dtype=np.uint8)         # code of +1.0
    got = orc.dequant_block128(ones, s)
    assert np.array_equal(got, np.kron(s.astype(np.float64), np.ones((128, 128))))
    neg = np.full((256, 384), 0xB8, dtype=np.uint8)          # code of -1.0
    assert np.array_equal(orc.dequant_block128(neg, s), -got)


def test_dequant_random_codes_match_torch_scaled_decode():
    rng = np.random.default_rng(1)
    q = rng.integers(0, 256, size=(256, 128), dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x00                             # no NaN codes
    s = np.array([[0.25], [3.0]], dtype=np.float32)
    got = orc.dequant_block128(q, s)
    dec = torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(got[:128], dec[:128] * 0.25)
    assert np.array_equal(got[128:], dec[128:] * np.float64(np.float32(3.0)))


# ---------------------------------------------------------------- router logits
#
# The gate ("Wide Expert Parallelism", section "What is an MoE layer?") scores
# every expert for a token; the skewed workloads add a per-expert bias to those
# scores, which moves both the choice and the gate values.  Two pins of
# ``router_logits``: torch's own affine map in float64 (a different routine),
# on a problem with T == E so that a bias added along the token axis would
# broadcast silently instead of raising; and a hand-worked example whose bias
# changes the chosen experts of one token and the gate values of another.


def _pin_router_against_torch_linear(fn):
    rng = np.random.default_rng(11)
    T = E = 12
    d = 20
    x = rng.standard_normal((T, d))
    w = rng.standard_normal((d, E))
    b = rng.standard_normal(E) * 3.0
    ref = Fnn.linear(torch.from_numpy(x), torch.from_numpy(np.ascontiguousarray(w.T)),
                     torch.from_numpy(b)).numpy()
    got = np.asarray(fn(x, w, b), dtype=np.float64)
    assert got.shape == (T, E)
    assert np.allclose(got, ref, rtol=1e-13, atol=1e-13)
    # no bias means a zero bias
    ref0 = Fnn.linear(torch.from_numpy(x), torch.from_numpy(np.ascontiguousarray(w.T))).numpy()
    assert np.allclose(np.asarray(fn(x, w, None), dtype=np.float64), ref0, rtol=1e-13, atol=1e-13)


def _pin_router_hand_example(fn):
    # d = 2, E = 3: W_r picks the token's first and second feature as the
    # scores of experts 0 and 1; expert 2 scores 0 before its bias of 2.5.
    w = np.array([[1.0, 0.0, 0.0],
                  [0.0, 1.0, 0.0]])
    b = np.array([0.0, 0.0, 2.5])
    x = np.array([[1.0, 2.0],     # scores 1, 2, 0 -> with bias 1, 2, 2.5
                  [3.0, 1.0]])    # scores 3, 1, 0 -> with bias 3, 1, 2.5
    L = np.asarray(fn(x, w, b), dtype=np.float64)
    assert np.array_equal(L, [[1.0, 2.0, 2.5], [3.0, 1.0, 2.5]])
    idx = orc.topk_select(L, 2)
    gates = orc.renormalised_gates(L, idx)
    sig = lambda z: 1.0 / (1.0 + math.exp(-z))  # k = 2: the gates are logistic
    # token 0: the bias lifts expert 2 over expert 0 (unbiased top-2: 1, 0)
    assert idx[0].tolist() == [2, 1]
    assert np.allclose(gates[0], [sig(0.5), sig(-0.5)], rtol=0, atol=1e-15)
    # token 1: expert 2 replaces expert 1, and the gate of expert 0 drops from
    # sigmoid(3 - 1) to sigmoid(3 - 2.5)
    assert idx[1].tolist() == [0, 2]
    assert np.allclose(gates[1], [sig(0.5), sig(-0.5)], rtol=0, atol=1e-15)


def test_router_logits_match_torch_linear_with_bias():
    _pin_router_against_torch_linear(orc.router_logits)


def test_router_bias_moves_selection_and_gates_hand_example():
    _pin_router_hand_example(orc.router_logits)


@pytest.mark.parametrize("slip", ["bias dropped", "bias negated", "bias on the token axis",
                                  "bias added twice", "router matrix transposed"])
def test_router_pins_catch_planted_slips(slip):
    """Mistakes planted in a copy of the oracle's logit formula (on the CPU)
    must fail at least one of the two pins above."""
    def slipped(x, w, b):
        b = None if b is None else np.asarray(b, dtype=np.float64)
        if slip == "router matrix transposed":
            L = x @ w.T if w.shape[0] == w.shape[1] else (x @ w)[:, ::-1]
        else:
            L = x @ w
        if b is None or slip == "bias dropped":
            return L
        if slip == "bias negated":
            return L - b[None, :]
        if slip == "bias on the token axis":
            return L + b[:, None] if L.shape[0] == L.shape[1] else L + b[None, ::-1]
        if slip == "bias added twice":
            return L + 2 * b[None, :]
        return L + b[None, :]

    failed = 0
    for pin in (_pin_router_against_torch_linear, _pin_router_hand_example):
        try:
            pin(slipped)
        except AssertionError:
            failed += 1
    assert failed >= 1, f"planted slip '{slip}' passed every router pin"


# ---------------------------------------------------------------- routing

@pytest.mark.parametrize("T,E,k,levels", [(40, 8, 2, 3), (30, 16, 5, 4), (25, 6, 6, 2), (20, 12, 1, 2)])
def test_topk_matches_rank_definition_with_ties(T, E, k, levels):
    rng = np.random.default_rng(T * 100 + E)
    L = (rng.integers(0, levels, size=(T, E)) * 0.5).astype(np.float32)
    idx = orc.topk_select(L, k)
    for t in range(T):
        # e is chosen iff fewer than k experts beat it under (-L, e)
        chosen = set()
        for e in range(E):
            beaters = sum(1 for f in range(E) if L[t, f] > L[t, e] or (L[t, f] == L[t, e] and f < e))
            if beaters < k:
                chosen.add(e)
        assert set(idx[t].tolist()) == chosen
        keys = [(-float(L[t, e]), int(e)) for e in idx[t]]
        assert keys == sorted(keys)


def test_topk_all_equal_logits_pick_lowest_indices():
    L = np.zeros((5, 9), dtype=np.float32)
    assert np.array_equal(orc.topk_select(L, 4), np.tile(np.arange(4, dtype=np.int32), (5, 1)))


def test_topk_max_over_subsets_brute_force():
    # the chosen set has the largest logit sum among all k-subsets (distinct logits)
    rng = np.random.default_rng(2)
    L = rng.standard_normal((10, 7)).astype(np.float32)
    idx = orc.topk_select(L, 3)
    for t in range(10):
        best = max(itertools.combinations(range(7), 3), key=lambda c: sum(float(L[t, e]) for e in c))
        assert set(idx[t].tolist()) == set(best)


def test_topk_orders_nan_as_minus_inf_hand_example():
    # The pages are silent on non-finite logits; the contract reads a NaN as
    # -inf, so NaN and -inf tie below every finite logit (lower index first)
    # and +inf ranks above them.
    L = np.array([[np.nan, 1.0, -np.inf, 0.5, np.nan, np.inf],
                  [np.nan, np.nan, np.nan, np.nan, np.nan, np.nan],
                  [-np.inf, np.nan, -np.inf, -2.0, np.nan, -1.0]], dtype=np.float32)
    assert orc.topk_select(L, 6).tolist() == [[5, 1, 3, 0, 2, 4],
                                              [0, 1, 2, 3, 4, 5],
                                              [5, 3, 0, 1, 2, 4]]


def test_gates_k2_equal_logistic_of_difference():
    rng = np.random.default_rng(3)
    L = rng.standard_normal((50, 8)) * 3
    idx = orc.topk_select(L, 2)
    w = orc.renormalised_gates(L, idx)
    l0 = np.take_along_axis(L, idx[:, :1].astype(np.int64), 1)[:, 0]
    l1 = np.take_along_axis(L, idx[:, 1:2].astype(np.int64), 1)[:, 0]
    assert np.allclose(w[:, 0], scipy.special.expit(l0 - l1), rtol=0, atol=1e-15)
    assert np.allclose(w[:, 1], scipy.special.expit(l1 - l0), rtol=0, atol=1e-15)


def test_gates_k_equal_E_is_full_softmax():
    rng = np.random.default_rng(4)
    L = rng.standard_normal((30, 6)) * 4
    idx = orc.topk_select(L, 6)
    w = orc.renormalised_gates(L, idx)
    p = scipy.special.softmax(L, axis=1)
    assert np.allclose(w, np.take_along_axis(p, idx.astype(np.int64), 1), rtol=0, atol=1e-15)


def test_gates_sum_to_one_and_shift_invariant():
    rng = np.random.default_rng(5)
    L = rng.standard_normal((100, 32)) * 5
    idx = orc.topk_select(L, 8)
    w = orc.renormalised_gates(L, idx)
    assert np.abs(w.sum(1) - 1).max() <= 1e-15
    assert (np.diff(w, axis=1) <= 0).all()          # listed by descending logit
    w2 = orc.renormalised_gates(L + 7.25, idx)
    assert np.allclose(w, w2, rtol=0, atol=1e-15)


# ---------------------------------------------------------------- permutation

@pytest.mark.parametrize("T,E,k,e0,E_l", [(64, 8, 2, 0, 8), (200, 32, 4, 8, 8), (50, 16, 16, 0, 16),
                                          (33, 10, 3, 9, 1), (1, 4, 2, 0, 4)])
def test_permutation_matches_stable_argsort_and_invariants(T, E, k, e0, E_l):
    rng = np.random.default_rng(T + E)
    L = rng.standard_normal((T, E)).astype(np.float32)
    idx = orc.topk_select(L, k)
    counts, offsets, sorted_slot, slot_pos = orc.expert_permutation(idx, e0, E_l)
    flat = idx.reshape(-1).astype(np.int64)
    keep = (flat >= e0) & (flat < e0 + E_l)
    # library routines: bincount and a stable argsort
    assert np.array_equal(counts, np.bincount(flat[keep] - e0, minlength=E_l))
    ks = np.nonzero(keep)[0]
    assert np.array_equal(sorted_slot, ks[np.argsort(flat[ks] - e0, kind="stable")])
    # conservation, bijection, -1 exactly on dropped slots
    assert offsets[0] == 0 and offsets[-1] == counts.sum() == keep.sum()
    if e0 == 0 and E_l == E:
        assert counts.sum() == T * k
    assert np.array_equal(slot_pos[sorted_slot], np.arange(sorted_slot.size))
    assert np.array_equal(slot_pos < 0, ~keep)
    # segments: expert id non-decreasing, slot strictly increasing inside
    ex = flat[sorted_slot]
    assert (np.diff(ex) >= 0).all()
    same = np.diff(ex) == 0
    assert (np.diff(sorted_slot)[same] > 0).all()


def test_mean_expert_load_matches_page_figure():
    g = json.load(open(GOLDEN))["mean_expert_load"]
    E, k, B = g["E"], g["k"], g["B"]
    rng = np.random.default_rng(6)
    L = rng.standard_normal((B, E)).astype(np.float32)
    counts, offsets, _, _ = orc.expert_permutation(orc.topk_select(L, k), 0, E)
    assert counts.sum() / E == g["mean_tokens_per_expert"]
    assert offsets[-1] == B * k


# ---------------------------------------------------------------- experts / combine

def test_silu_matches_torch():
    z = np.linspace(-800, 800, 20001)
    ref = Fnn.silu(torch.from_numpy(z)).numpy()
    assert np.allclose(orc.silu(z), ref, rtol=1e-15, atol=1e-300)


def test_e1_k1_reduces_to_dense_swiglu_ffn():
    rng = np.random.default_rng(7)
    x, L, wg, wu, wd = _f32_problem(rng, T=20, d=16, E=1, k=1, F=24)
    r = orc.moe_layer_forward(x, L, 1, wg, wu, wd, act_fmt="f32", weight_fmt="f32")
    assert np.array_equal(r["topk_w"], np.ones((20, 1)))
    X = torch.from_numpy(x.astype(np.float64))
    Wg, Wu, Wd = (torch.from_numpy(a[0].astype(np.float64)) for a in (wg, wu, wd))
    ref = (Fnn.silu(X @ Wg.T) * (X @ Wu.T)) @ Wd.T
    assert np.allclose(r["out"], ref.numpy(), rtol=1e-12, atol=1e-13)


def test_swiglu_gate_and_up_are_not_swapped():
    # d = 1, x = 1: the gate pre-activation is 40 for every column, where
    # silu(40) = 40 to double precision, so out = 40 * sum_f u_f v_f exactly
    F = 4
    u = np.array([0.5, -1.0, 2.0, 0.25], dtype=np.float32)
    v = np.array([1.0, 3.0, -0.5, 2.0], dtype=np.float32)
    x = np.ones((1, 1), dtype=np.float32)
    wg = np.full((1, F, 1), 40.0, dtype=np.float32)
    wu = u.reshape(1, F, 1)
    wd = v.reshape(1, 1, F)
    r = orc.moe_layer_forward(x, np.zeros((1, 1), np.float32), 1, wg, wu, wd,
                              act_fmt="f32", weight_fmt="f32")
    assert r["out"][0, 0] == pytest.approx(40.0 * float(np.dot(u, v)), rel=1e-15)
    # and a zero gate pre-activation gives silu(0) = 0 whatever the up projection
    r0 = orc.moe_layer_forward(x, np.zeros((1, 1), np.float32), 1, np.zeros_like(wg), wu, wd,
                               act_fmt="f32", weight_fmt="f32")
    assert r0["out"][0, 0] == 0.0


def test_identical_experts_give_dense_ffn_for_any_routing():
    rng = np.random.default_rng(8)
    x, L, wg, wu, wd = _f32_problem(rng, T=24, d=16, E=6, k=3, F=32, bias=True)
    wg[:] = wg[0]
    wu[:] = wu[0]
    wd[:] = wd[0]
    r = orc.moe_layer_forward(x, L, 3, wg, wu, wd, act_fmt="f32", weight_fmt="f32")
    dense = orc.swiglu_ffn(x.astype(np.float64), wg[0].T.astype(np.float64),
                           wu[0].T.astype(np.float64), wd[0].T.astype(np.float64))
    assert np.allclose(r["out"], dense, rtol=1e-12, atol=1e-13)


def test_k_equal_E_is_softmax_weighted_mixture():
    rng = np.random.default_rng(9)
    T, d, E, F = 12, 8, 5, 16
    x, L, wg, wu, wd = _f32_problem(rng, T=T, d=d, E=E, k=E, F=F)
    r = orc.moe_layer_forward(x, L, E, wg, wu, wd, act_fmt="f32", weight_fmt="f32")
    p = scipy.special.softmax(L.astype(np.float64), axis=1)
    X = torch.from_numpy(x.astype(np.float64))
    ref = torch.zeros((T, d), dtype=torch.float64)
    for e in range(E):
        Wg, Wu, Wd = (torch.from_numpy(a[e].astype(np.float64)) for a in (wg, wu, wd))
        ref += torch.from_numpy(p[:, e:e + 1]) * ((Fnn.silu(X @ Wg.T) * (X @ Wu.T)) @ Wd.T)
    assert np.allclose(r["out"], ref.numpy(), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("T,d,E,k,F,e0,E_l", [(64, 128, 8, 2, 256, 0, 8), (16, 8, 8, 3, 16, 0, 8),
                                              (9, 4, 5, 5, 8, 0, 5), (13, 16, 7, 1, 8, 2, 3),
                                              (11, 8, 4, 2, 8, 0, 4)])
def test_brute_force_dense_masked_evaluation_agrees(T, d, E, k, F, e0, E_l):
    rng = np.random.default_rng(T * d + E)
    x, L, wg, wu, wd = _f32_problem(rng, T, d, E, k, F, E_l=E_l, e0=e0, bias=True)
    r = orc.moe_layer_forward(x, L, k, wg, wu, wd, act_fmt="f32", weight_fmt="f32", e0=e0, E_l=E_l)
    bf = orc.brute_force_dense(x, L, k, wg, wu, wd, act_fmt="f32", weight_fmt="f32", e0=e0, E_l=E_l)
    assert np.linalg.norm(r["out"] - bf) <= 1e-12 * max(np.linalg.norm(bf), 1e-300)


def test_token_permutation_equivariance():
    rng = np.random.default_rng(10)
    x, L, wg, wu, wd = _f32_problem(rng, T=30, d=8, E=6, k=2, F=16)
    perm = rng.permutation(30)
    a = orc.moe_layer_forward(x, L, 2, wg, wu, wd, act_fmt="f32", weight_fmt="f32")
    b = orc.moe_layer_forward(x[perm], L[perm], 2, wg, wu, wd, act_fmt="f32", weight_fmt="f32")
    assert np.array_equal(a["topk_idx"][perm], b["topk_idx"])
    assert np.allclose(a["out"][perm], b["out"], rtol=1e-13, atol=1e-14)


def test_power_of_two_scaling_of_down_projection_is_exact():
    rng = np.random.default_rng(11)
    x, L, wg, wu, wd = _f32_problem(rng, T=16, d=8, E=4, k=2, F=8)
    a = orc.moe_layer_forward(x, L, 2, wg, wu, wd, act_fmt="f32", weight_fmt="f32")
    b = orc.moe_layer_forward(x, L, 2, wg, wu, wd * np.float32(2), act_fmt="f32", weight_fmt="f32")
    assert np.array_equal(2 * a["out"], b["out"])


def test_expert_parallel_blocks_sum_to_the_whole_layer():
    # the per-rank partial outputs of E/4 experts each add up to the full layer
    rng = np.random.default_rng(12)
    T, d, E, k, F = 40, 8, 16, 4, 16
    x, L, wg, wu, wd = _f32_problem(rng, T, d, E, k, F, bias=True)
    full = orc.moe_layer_forward(x, L, k, wg, wu, wd, act_fmt="f32", weight_fmt="f32")
    tot = np.zeros_like(full["out"])
    kept = 0
    for r in range(4):
        sl = slice(4 * r, 4 * r + 4)
        part = orc.moe_layer_forward(x, L, k, wg[sl], wu[sl], wd[sl], act_fmt="f32",
                                     weight_fmt="f32", e0=4 * r, E_l=4)
        tot += part["out"]
        kept += int(part["offsets"][-1])
        # tokens with no slot in this block get exactly zero
        none = ~((part["topk_idx"] >= 4 * r) & (part["topk_idx"] < 4 * r + 4)).any(1)
        assert (part["out"][none] == 0).all()
    assert kept == T * k
    assert np.allclose(tot, full["out"], rtol=1e-13, atol=1e-14)


def test_sampled_tokens_equal_full_rows():
    rng = np.random.default_rng(13)
    x, L, wg, wu, wd = _f32_problem(rng, T=50, d=8, E=8, k=3, F=16)
    full = orc.moe_layer_forward(x, L, 3, wg, wu, wd, act_fmt="f32", weight_fmt="f32")
    toks = np.array([3, 0, 49, 17])
    part = orc.moe_layer_forward(x, L, 3, wg, wu, wd, act_fmt="f32", weight_fmt="f32", tokens=toks)
    # same arithmetic, only the BLAS blocking of the row count differs
    assert np.allclose(part["out"], full["out"][toks], rtol=1e-13, atol=1e-15)


def test_bf16_and_fp8_paths_equal_the_f32_path_on_shared_values():
    # weights whose values are exactly representable in all three formats
    # (small integers times powers of two) give identical oracle outputs, so
    # the format plumbing (bit decode, fp8 table and scale blocks) is right
    rng = np.random.default_rng(14)
    E_l, F, d, T, k = 2, 128, 256, 8, 1
    vals = np.array([0, 0.5, 1, 1.5, 2, -0.5, -1, -2, 0.25, -0.125], dtype=np.float32)
    wg = rng.choice(vals, size=(E_l, F, d)).astype(np.float32)
    wu = rng.choice(vals, size=(E_l, F, d)).astype(np.float32)
    wd = rng.choice(vals, size=(E_l, d, F)).astype(np.float32)
    x = rng.choice(vals, size=(T, d)).astype(np.float32)
    L = rng.standard_normal((T, E_l)).astype(np.float32)
    ref = orc.moe_layer_forward(x, L, k, wg, wu, wd, act_fmt="f32", weight_fmt="f32")["out"]

    def bf(a):
        return torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got_bf = orc.moe_layer_forward(bf(x), L, k, bf(wg), bf(wu), bf(wd), act_fmt="bf16",
                                   weight_fmt="bf16")["out"]
    assert np.array_equal(got_bf, ref)

    # fp8: store w / 2^j with scale 2^j, j varying per block
    def q8(a, blocks):
        s = np.exp2(rng.integers(-2, 3, size=(a.shape[0],) + blocks)).astype(np.float32)
        big = np.stack([np.kron(s[j], np.ones((128, 128), np.float32)) for j in range(a.shape[0])])
        q = torch.from_numpy(a / big).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        return q, s
    qg, sg = q8(wg, (1, 2))
    qu, su = q8(wu, (1, 2))
    qd, sd = q8(wd, (2, 1))
    got8 = orc.moe_layer_forward(bf(x), L, k, qg, qu, qd, act_fmt="bf16", weight_fmt="fp8",
                                 s_gate=sg, s_up=su, s_down=sd)["out"]
    assert np.array_equal(got8, ref)
