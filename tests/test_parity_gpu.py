"""Parity of the HIP library (through the C ABI) with the float64 CPU oracle.

Routing, counts, offsets, the permutation and slot positions must be equal bit
for bit, given the library's own float32 logits (both sides decide on the same
numbers; ties go to the lower expert index).  Gates must agree within 1e-6
absolute, logits within 1e-5 relative L2 of the float64 logits, and the layer
output within a relative L2 error of 1e-5 (float32), 1e-2 (bf16, and bf16
activations with MXFP4 weights, which are widened exactly) or 3e-2 (bf16
activations with FP8-E4M3 weights).  At the full workload sizes the output is
compared on a seeded sample of tokens that the oracle evaluates one by one.
"""
import numpy as np
import pytest
import torch

from mixture_experts_layer_15_amd import binding as B
from mixture_experts_layer_15_amd import synth
from oracle import moe_oracle as orc

pytestmark = pytest.mark.gpu

TOL = {("f32", "f32"): 1e-5, ("bf16", "bf16"): 1e-2, ("bf16", "fp8"): 3e-2,
       ("bf16", "mxfp4"): 1e-2}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load_library()


DEV = "cuda"


def _prob(wl, blocked=False):
    return B.problem(wl.T, wl.d, wl.E, wl.k, wl.F, wl.expert_begin, wl.num_local, wl.act, wl.weight,
                     blocked=blocked)


def upload(pr):
    g = {}
    for n in ("x", "w_router", "bias", "w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down"):
        t = getattr(pr, n)
        g[n] = None if t is None else t.to(DEV)
    return g


def forward(pr, g=None, logits_in=None, blocked=False):
    """moe_forward with every optional output requested; returns CPU tensors.
    blocked: g holds the weights in the blocked layout (see pack())."""
    wl = pr.wl
    g = upload(pr) if g is None else g
    T, d, E, k, El = wl.T, wl.d, wl.E, wl.k, wl.num_local
    p = _prob(wl, blocked)
    o = dict(
        out=torch.empty((T, d), dtype=pr.x.dtype, device=DEV),
        logits=(logits_in.to(DEV) if logits_in is not None
                else torch.empty((T, E), dtype=torch.float32, device=DEV)),
        topk_idx=torch.empty((T, k), dtype=torch.int32, device=DEV),
        topk_w=torch.empty((T, k), dtype=torch.float32, device=DEV),
        counts=torch.empty((El,), dtype=torch.int32, device=DEV),
        offsets=torch.empty((El + 1,), dtype=torch.int32, device=DEV),
        sorted_slot=torch.empty((T * k,), dtype=torch.int32, device=DEV),
        slot_pos=torch.empty((T * k,), dtype=torch.int32, device=DEV),
    )
    ws = B.workspace(p, B.MOE_CALL_FORWARD, DEV)
    B.moe_forward(p, x=g["x"], w_router=None if logits_in is not None else g["w_router"],
                  router_bias=g["bias"], w_gate=g["w_gate"], w_up=g["w_up"], w_down=g["w_down"],
                  s_gate=g["s_gate"], s_up=g["s_up"], s_down=g["s_down"], ws=ws, **o)
    torch.cuda.synchronize()
    return {n: t.cpu() for n, t in o.items()}


def pack(pr, g):
    """A copy of the uploaded problem with the expert weights in the library's
    blocked layout (moe_pack_weights)."""
    wl = pr.wl
    p = _prob(wl)
    out = dict(g)
    for n, which in (("w_gate", 0), ("w_up", 0), ("w_down", 1)):
        dst = torch.empty_like(g[n])
        B.moe_pack_weights(p, which, g[n], dst)
        out[n] = dst
    torch.cuda.synchronize()
    return out


def oracle_for(pr, logits, tokens=None):
    wl = pr.wl
    return orc.moe_layer_forward(
        synth.raw(pr.x), logits.numpy(), wl.k, synth.raw(pr.w_gate), synth.raw(pr.w_up),
        synth.raw(pr.w_down), act_fmt=wl.act, weight_fmt=wl.weight, e0=wl.expert_begin,
        E_l=wl.num_local, s_gate=synth.raw(pr.s_gate), s_up=synth.raw(pr.s_up),
        s_down=synth.raw(pr.s_down), tokens=tokens)


def rel_l2(got, ref):
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return np.linalg.norm(np.asarray(got, dtype=np.float64) - ref) / (den if den > 0 else 1.0)


def check(pr, gpu, tokens=None, check_logits=True):
    wl = pr.wl
    ref = oracle_for(pr, gpu["logits"], tokens)
    N = int(ref["offsets"][-1])
    # routing and dispatch: bit-exact
    assert np.array_equal(gpu["topk_idx"].numpy(), ref["topk_idx"]), "topk_idx"
    assert np.array_equal(gpu["counts"].numpy(), ref["counts"]), "counts"
    assert np.array_equal(gpu["offsets"].numpy(), ref["offsets"]), "offsets"
    assert np.array_equal(gpu["sorted_slot"].numpy()[:N], ref["sorted_slot"]), "sorted_slot"
    assert np.array_equal(gpu["slot_pos"].numpy(), ref["slot_pos"]), "slot_pos"
    # gates
    gw = gpu["topk_w"].numpy().astype(np.float64)
    assert np.abs(gw - ref["topk_w"]).max() <= 1e-6
    assert np.abs(gw.sum(1) - 1).max() <= 1e-6
    # logits against float64 from the same stored inputs
    if check_logits and pr.w_router is not None:
        L64 = orc.router_logits(orc.decode_act(synth.raw(pr.x), wl.act),
                                orc.decode_act(synth.raw(pr.w_router), wl.act),
                                None if pr.bias is None else pr.bias.numpy())
        assert rel_l2(gpu["logits"].numpy(), L64) <= 1e-5, "logits"
    # output: the relative L2 error over all compared rows, and over every row
    # on its own (a few wrong rows, or one wrong element of a row, cannot hide
    # in the global norm); rows the oracle gives as 0 (no local slot) must be
    # exactly 0
    got = gpu["out"].float().numpy()[ref["tokens"]].astype(np.float64)
    err = rel_l2(got, ref["out"])
    tol = TOL[(wl.act, wl.weight)]
    row_ref = np.linalg.norm(ref["out"], axis=1)
    row_diff = np.linalg.norm(got - ref["out"], axis=1)
    zero = row_ref == 0
    assert np.all(got[zero] == 0), "rows without a local slot must be 0"
    worst = float((row_diff[~zero] / row_ref[~zero]).max()) if (~zero).any() else 0.0
    print(f"[{wl.name}] N={N} out rel L2 = {err:.3e}, worst row {worst:.3e} (tol {tol:g})",
          flush=True)
    assert err <= tol
    assert worst <= tol, f"row relative L2 {worst:.3e}"
    if wl.weight == "fp8":
        # FP8 weights are widened exactly to bf16 and their block scales folded
        # into float32 sums: the same numerics as bf16 weights, so the bf16 bound
        # holds as well as the looser fp8 one
        assert err <= TOL[("bf16", "bf16")] and worst <= TOL[("bf16", "bf16")]
    return ref, err


SMALL = {
    # tiny fp32 workload at its real size
    "tiny": synth.WORKLOADS["tiny"],
    # few rows per expert (32-row tiles): several N tiles, ragged segments
    "bf16_decode_tiles": synth.WORKLOADS["decode"].replace(
        name="bf16_T200_d256_E16_k4_F384", T=200, d=256, E=16, num_local=16, k=4, F=384, seed=21),
    # many rows per expert (128-row tiles), ragged tails, d not a multiple of 256
    "bf16_prefill_tiles": synth.WORKLOADS["prefill"].replace(
        name="bf16_T700_d384_E8_k2_F256", T=700, d=384, E=8, num_local=8, k=2, F=256, seed=22),
    # skewed prefill-like with bias, down tile clipped in N
    "bf16_skew": synth.WORKLOADS["prefill"].replace(
        name="bf16_T1000_d640_E32_k4_F512_zipf", T=1000, d=640, E=32, num_local=32, k=4, F=512,
        seed=23),
    # FP8 weights on an expert-parallel rank block (experts 8..15 of 32)
    "fp8_rank_decode": synth.WORKLOADS["dsv3_rank"].replace(
        name="fp8_T100_d256_E32_local8-15_k4_F256", T=100, d=256, E=32, num_local=8,
        expert_begin=8, k=4, F=256, seed=24),
    "fp8_rank_prefill": synth.WORKLOADS["dsv3_rank"].replace(
        name="fp8_T2000_d512_E16_local0-7_k4_F384", T=2000, d=512, E=16, num_local=8,
        expert_begin=0, k=4, F=384, seed=25),
    # more than 8192 slots: the multi-workgroup permutation, ragged last chunk
    "bf16_many_slots": synth.WORKLOADS["prefill"].replace(
        name="bf16_T3001_d256_E64_k4_F256_zipf", T=3001, d=256, E=64, num_local=64, k=4, F=256,
        seed=27),
    # the same on an expert-parallel block (many slots dropped)
    "fp8_many_slots_rank": synth.WORKLOADS["dsv3_rank"].replace(
        name="fp8_T2500_d256_E64_local48-63_k6_F256", T=2500, d=256, E=64, num_local=16,
        expert_begin=48, k=6, F=256, seed=28),
    # >= 1024 rows per expert: 256 x 256 tiles, N tiles clipped in both GEMMs
    "bf16_big_tiles": synth.WORKLOADS["mixtral"].replace(
        name="bf16_T2100_d384_E4_k2_F384_gauss", T=2100, d=384, E=4, num_local=4, k=2, F=384,
        seed=29),
    # many tokens and more than 128 experts: router logits from the GEMM
    # pipeline (E not a multiple of 16, then not of 4: masked logit columns)
    "bf16_router_gemm": synth.WORKLOADS["prefill"].replace(
        name="bf16_T1100_d384_E200_k6_F128_zipf", T=1100, d=384, E=200, num_local=200, k=6,
        F=128, seed=30),
    # many tokens, E = 100 (not a multiple of 8): the staged router product
    # with masked expert columns, top-k rows with padded lanes
    "bf16_router_direct_E100": synth.WORKLOADS["prefill"].replace(
        name="bf16_T1100_d256_E100_k4_F128_zipf", T=1100, d=256, E=100, num_local=100, k=4,
        F=128, seed=38),
    # more than 256 experts: router top-k rows of 32 keys per lane
    "bf16_router_E320": synth.WORKLOADS["prefill"].replace(
        name="bf16_T1040_d256_E320_k5_F128_zipf", T=1040, d=256, E=320, num_local=320, k=5,
        F=128, seed=37),
    "bf16_router_gemm_odd_E": synth.WORKLOADS["prefill"].replace(
        name="bf16_T1030_d256_E130_k3_F128_zipf", T=1030, d=256, E=130, num_local=130, k=3,
        F=128, seed=32),
    # the router GEMM with its K range cut into parts (35 tiles of 32 tokens,
    # 4 parts), summed in part order by the top-k kernel
    "bf16_router_gemm_ksplit": synth.WORKLOADS["prefill"].replace(
        name="bf16_T1100_d2048_E200_k6_F128_zipf", T=1100, d=2048, E=200, num_local=200, k=6,
        F=128, seed=78),
    # many tokens: the router GEMM on 256 x 256 tiles, ragged last token tile,
    # E not a multiple of 16, K cut into parts
    "bf16_router_gemm_big": synth.WORKLOADS["prefill"].replace(
        name="bf16_T8200_d1024_E170_k4_F128_zipf", T=8200, d=1024, E=170, num_local=170, k=4,
        F=128, seed=79),
    # MXFP4 weights: decode tiles (ragged N tiles of 128 features), and the
    # 128 x 512 tiles on an expert-parallel block with a half-filled N tile
    "mxfp4_decode_tiles": synth.WORKLOADS["decode_mxfp4"].replace(
        name="mxfp4_T200_d256_E16_k4_F384", T=200, d=256, E=16, num_local=16, k=4, F=384, seed=33),
    # decode tiles on an expert-parallel block with d and F not multiples of
    # 256 (bf16 and MXFP4)
    "bf16_decode_rank": synth.WORKLOADS["decode"].replace(
        name="bf16_T50_d384_E24_local6-17_k3_F640", T=50, d=384, E=24, num_local=12,
        expert_begin=6, k=3, F=640, seed=35),
    "mxfp4_decode_rank": synth.WORKLOADS["decode_mxfp4"].replace(
        name="mxfp4_T60_d384_E24_local6-17_k3_F640", T=60, d=384, E=24, num_local=12,
        expert_begin=6, k=3, F=640, seed=36),
    "mxfp4_prefill_rank": synth.WORKLOADS["decode_mxfp4"].replace(
        name="mxfp4_T2000_d512_E16_local4-11_k4_F384_zipf", T=2000, d=512, E=16, num_local=8,
        expert_begin=4, k=4, F=384, bias=("zipf", 1.1, 2.0), seed=34, regime="prefill"),
    # f32 with more tiles than the tiny workload
    "f32_tiles": synth.WORKLOADS["tiny"].replace(
        name="f32_T300_d256_E8_k3_F384", T=300, d=256, E=8, num_local=8, k=3, F=384, seed=26),
    # f32 router product over two expert passes (150 experts: the second pass
    # masked past E) and four K splits
    "f32_router_E150": synth.WORKLOADS["tiny"].replace(
        name="f32_T100_d512_E150_k4_F128", T=100, d=512, E=150, num_local=150, k=4, F=128,
        seed=39),
}


@pytest.mark.parametrize("case", list(SMALL))
def test_small_full_parity(case):
    pr = synth.make_problem(SMALL[case])
    check(pr, forward(pr))


# Cases whose GEMMs run every tile plan with long K loops (at least 8 K stages,
# so the next item's stages are loaded inside the running item's K loop).
# Capping the persistent grid at 8 workgroups gives each workgroup many items.
MULTI = {
    "decode_plan": synth.WORKLOADS["decode"].replace(
        name="bf16_T40_d512_E16_k4_F512", T=40, d=512, E=16, num_local=16, k=4, F=512, seed=60),
    "decode64_plan": synth.WORKLOADS["decode"].replace(
        name="bf16_T96_d512_E16_k4_F512", T=96, d=512, E=16, num_local=16, k=4, F=512, seed=61),
    "wide_plan": synth.WORKLOADS["prefill"].replace(
        name="bf16_T900_d512_E8_k2_F384_zipf", T=900, d=512, E=8, num_local=8, k=2, F=384,
        seed=62),
    "big_plan": synth.WORKLOADS["mixtral"].replace(
        name="bf16_T2300_d512_E4_k2_F512_gauss", T=2300, d=512, E=4, num_local=4, k=2, F=512,
        seed=63),
    "fp8_plan": synth.WORKLOADS["dsv3_rank"].replace(
        name="fp8_T1500_d512_E16_local4-11_k4_F512", T=1500, d=512, E=16, num_local=8,
        expert_begin=4, k=4, F=512, seed=64),
    "fp8_decode_plan": synth.WORKLOADS["dsv3_rank"].replace(
        name="fp8_T64_d512_E32_local0-15_k4_F512", T=64, d=512, E=32, num_local=16,
        expert_begin=0, k=4, F=512, seed=65),
    "mxfp4_decode_plan": synth.WORKLOADS["decode_mxfp4"].replace(
        name="mxfp4_T40_d512_E16_k4_F512", T=40, d=512, E=16, num_local=16, k=4, F=512, seed=68),
    "mxfp4_plan": synth.WORKLOADS["decode_mxfp4"].replace(
        name="mxfp4_T1500_d512_E16_local4-11_k4_F512", T=1500, d=512, E=16, num_local=8,
        expert_begin=4, k=4, F=512, seed=69, regime="prefill"),
}


@pytest.mark.parametrize("case", list(MULTI))
def test_many_items_per_workgroup(case, monkeypatch):
    pr = synth.make_problem(MULTI[case])
    g = upload(pr)
    wide = forward(pr, g)
    monkeypatch.setenv("MOE_MI355X_MAX_WORKGROUPS", "8")
    narrow = forward(pr, g)
    # the same tiles computed in another order: identical bits
    assert torch.equal(narrow["out"], wide["out"])
    check(pr, narrow)


# Prefill-sized tiles deal their items to one virtual worker per compute unit
# and cut each item of the last, partial wave along K into parts, whose
# float32 partial sums a second kernel adds in part order.  Cases with whole
# waves and a split tail (gate/up), and with only tail items (down), on each
# prefill tile plan: (tile rows, gate/up features per N tile, down columns
# per N tile).
TAIL = {
    "wide": (synth.WORKLOADS["prefill"].replace(
        name="bf16_T1056_d1024_E16_k4_F2048_tail", T=1056, d=1024, E=16, num_local=16, k=4,
        F=2048, seed=74, bias=()), 128, 256, 512),
    "big": (synth.WORKLOADS["mixtral"].replace(
        name="bf16_T4200_d1024_E4_k2_F1024_tail", T=4200, d=1024, E=4, num_local=4, k=2, F=1024,
        seed=75), 256, 128, 256),
    "fp8": (synth.WORKLOADS["dsv3_rank"].replace(
        name="fp8_T4200_d1024_E16_local0-7_k4_F1024_tail", T=4200, d=1024, E=16, num_local=8,
        expert_begin=0, k=4, F=1024, seed=76), 128, 256, 512),
    "mxfp4": (synth.WORKLOADS["decode_mxfp4"].replace(
        name="mxfp4_T2100_d1024_E16_k4_F1024_tail", T=2100, d=1024, E=16, num_local=16, k=4,
        F=1024, seed=77, regime="prefill"), 128, 256, 512),
}


@pytest.mark.parametrize("case", list(TAIL))
def test_tail_split_items(case, monkeypatch):
    """The split tail against the oracle (every token), and the same bits with
    the grid capped at 8 and 24 workgroups (each then runs many virtual
    workers' items and parts in turn)."""
    wl, bm, gu_cols, dn_cols = TAIL[case]
    pr = synth.make_problem(wl)
    g = upload(pr)
    full = forward(pr, g)
    # the case exercises what it is meant to: a split gate/up tail after
    # whole waves, and a down GEMM with fewer items than compute units
    vw = torch.cuda.get_device_properties(0).multi_processor_count // 8 * 8
    mt = int(sum((int(c) + bm - 1) // bm for c in full["counts"].numpy()))
    gu_items, dn_items = mt * (wl.F // gu_cols), mt * (wl.d // dn_cols)
    print(f"[{wl.name}] M tiles {mt}, gate/up items {gu_items}, down items {dn_items}, "
          f"virtual workers {vw}", flush=True)
    assert gu_items > vw and 0 < gu_items % vw <= vw // 2
    assert dn_items < vw
    # (a tail item is cut only where two parts of at least 8 K stages of 64
    # fit: K = d >= 1024 here)
    assert wl.d >= 2 * 8 * 64
    check(pr, full)
    for cap in ("8", "24"):
        monkeypatch.setenv("MOE_MI355X_MAX_WORKGROUPS", cap)
        assert torch.equal(forward(pr, g)["out"], full["out"]), cap


@pytest.mark.parametrize("case", ["fp8_plan", "fp8_decode_plan"])
def test_fp8_zero_and_spread_block_scales(case):
    """Block scales that vary by up to 2^16 along K and blocks whose scale is 0
    (their nonzero codes must contribute nothing): the kernels fold the scales
    by rescaling the accumulator from block to block."""
    pr = synth.make_problem(MULTI[case].replace(name=case + "_scales", seed=66))
    g = torch.Generator().manual_seed(67)
    for n in ("s_gate", "s_up", "s_down"):
        s = getattr(pr, n)
        f = torch.exp2(torch.randint(-8, 9, s.shape, generator=g).float())
        f[torch.rand(s.shape, generator=g) < 0.15] = 0.0
        setattr(pr, n, (s * f).contiguous())
    check(pr, forward(pr))


@pytest.mark.parametrize("case", ["fp8_plan", "fp8_decode_plan"])
def test_fp8_block_scales_at_the_ratio_bound(case):
    """Consecutive K blocks of every weight row block alternate between scales
    2^16 and 2^-16: the largest ratio (2^32) the contract allows between the
    nonzero scales one output feature meets along K.  The accumulator is
    rescaled by 2^32 and 2^-32 at every block boundary and must stay finite
    and exact enough for the tolerance."""
    pr = synth.make_problem(MULTI[case].replace(name=case + "_ratio_bound", seed=73))
    for n in ("s_gate", "s_up", "s_down"):
        s = getattr(pr, n)
        kb = torch.arange(s.shape[-1])
        f = torch.where(kb % 2 == 0, 2.0 ** 16, 2.0 ** -16).to(s.dtype)
        setattr(pr, n, (s * f).contiguous())
    gpu = forward(pr)
    assert torch.isfinite(gpu["out"].float()).all()
    check(pr, gpu)


def same_plan_when_blocked(wl):
    # decode-sized GEMMs sum the products in another order on the two layouts
    # (bf16: the gate/up K loop is rotated on row-major weights only; MXFP4:
    # wave-streamed 64-deep slices on blocked weights, staged 128-deep steps on
    # row-major ones), so only parity holds there
    decode = wl.T * wl.k <= 64 * wl.num_local
    return not (decode and wl.weight in ("bf16", "mxfp4"))


@pytest.mark.parametrize("case", list(MULTI))
def test_blocked_weight_layout(case, monkeypatch):
    """Weights converted once to the blocked layout (each staged block one
    contiguous run) give exactly the bits of the row-major layout on every
    tile plan that stages the same K steps, on the full grid and with many
    items per workgroup; parity with the oracle in every case."""
    pr = synth.make_problem(MULTI[case])
    g = upload(pr)
    gb = pack(pr, g)
    assert not torch.equal(gb["w_gate"], g["w_gate"])   # the layout did change
    rows = forward(pr, g)
    blocked = forward(pr, gb, blocked=True)
    if same_plan_when_blocked(pr.wl):
        for n in rows:
            assert torch.equal(rows[n], blocked[n]), n
    check(pr, blocked)
    monkeypatch.setenv("MOE_MI355X_MAX_WORKGROUPS", "8")
    assert torch.equal(forward(pr, gb, blocked=True)["out"], blocked["out"])


@pytest.mark.parametrize("case", ["mxfp4_decode_tiles", "mxfp4_decode_rank", "bf16_decode_rank"])
def test_blocked_weight_layout_decode_shapes(case, monkeypatch):
    """Blocked weights on the decode-sized cases (MXFP4: the wave-streamed
    GEMMs, whose items wrap around the grid when it is capped), d and F not
    multiples of 256, an expert-parallel block."""
    pr = synth.make_problem(SMALL[case])
    gb = pack(pr, upload(pr))
    blocked = forward(pr, gb, blocked=True)
    check(pr, blocked)
    monkeypatch.setenv("MOE_MI355X_MAX_WORKGROUPS", "3")
    assert torch.equal(forward(pr, gb, blocked=True)["out"], blocked["out"])


@pytest.mark.parametrize("case", ["mxfp4_plan", "mxfp4_decode_plan"])
def test_mxfp4_spread_scales(case):
    """E8M0 scales moved by up to 2^8 either way per (32-value block, row): a
    scale read for the wrong row or K block cannot pass."""
    pr = synth.make_problem(MULTI[case].replace(name=case + "_scales", seed=71))
    g = torch.Generator().manual_seed(72)
    for n in ("s_gate", "s_up", "s_down"):
        s = getattr(pr, n).to(torch.int32)
        s = (s + torch.randint(-8, 9, s.shape, generator=g, dtype=torch.int32)).clamp(0, 252)
        setattr(pr, n, s.to(torch.uint8).contiguous())
    check(pr, forward(pr))


@pytest.mark.parametrize("case", ["T1", "k_equals_E", "E1_k1", "E512_k8"])
def test_edge_shapes(case):
    base = synth.WORKLOADS["decode"]
    wl = {
        "T1": base.replace(name="T1", T=1, d=256, E=16, num_local=16, k=4, F=256),
        "k_equals_E": base.replace(name="k_eq_E", T=40, d=128, E=8, num_local=8, k=8, F=128),
        "E1_k1": base.replace(name="E1_k1", T=70, d=256, E=1, num_local=1, k=1, F=256),
        "E512_k8": base.replace(name="E512", T=96, d=256, E=512, num_local=512, k=8, F=128),
    }[case]
    pr = synth.make_problem(wl, seed=31)
    gpu = forward(pr)
    check(pr, gpu)
    if case == "E1_k1":
        assert torch.all(gpu["topk_w"] == 1.0)


# Decode-sized batches: 512 experts (top-k keys spread over 8 per lane), an
# expert count that is not a multiple of 8 (masked router columns), k = 16
# with a full 64-token batch, d = 128 (fewer K steps than the router's
# splits would like), an expert-parallel block; and moe_route alone gives the
# logits and routing of moe_forward bit for bit.
DECODE_ROUTE = {
    "E512_T32": synth.WORKLOADS["decode"].replace(name="fused_T32_d256_E512_k8_F128", T=32, d=256,
                                                  E=512, num_local=512, k=8, F=128, seed=101),
    "E300_T20": synth.WORKLOADS["prefill"].replace(name="fused_T20_d384_E300_k6_F128_zipf", T=20,
                                                   d=384, E=300, num_local=300, k=6, F=128,
                                                   seed=102),
    "k16_T64": synth.WORKLOADS["decode"].replace(name="fused_T64_d512_E64_k16_F256", T=64, d=512,
                                                 E=64, num_local=64, k=16, F=256, seed=103),
    "d128_T33": synth.WORKLOADS["decode"].replace(name="fused_T33_d128_E40_k3_F128", T=33, d=128,
                                                  E=40, num_local=40, k=3, F=128, seed=104),
    "rank_T64": synth.WORKLOADS["dsv3_rank"].replace(name="fused_fp8_T64_d512_E96_local32-63_k8_F256",
                                                     T=64, d=512, E=96, num_local=32,
                                                     expert_begin=32, k=8, F=256, seed=105),
}


@pytest.mark.parametrize("case", list(DECODE_ROUTE))
def test_decode_sized_routing_and_standalone_route(case):
    wl = DECODE_ROUTE[case]
    pr = synth.make_problem(wl)
    g = upload(pr)
    gpu = forward(pr, g)
    check(pr, gpu)
    p = _prob(wl)
    T, E, k = wl.T, wl.E, wl.k
    logits = torch.empty((T, E), dtype=torch.float32, device=DEV)
    idx = torch.empty((T, k), dtype=torch.int32, device=DEV)
    gw = torch.empty((T, k), dtype=torch.float32, device=DEV)
    B.moe_route(p, g["x"], g["w_router"], g["bias"], logits, idx, gw,
                B.workspace(p, B.MOE_CALL_ROUTE, DEV))
    torch.cuda.synchronize()
    assert torch.equal(logits.cpu(), gpu["logits"])
    assert torch.equal(idx.cpu(), gpu["topk_idx"]) and torch.equal(gw.cpu(), gpu["topk_w"])


def test_logits_input_mode_with_planted_ties():
    wl = synth.WORKLOADS["decode"].replace(name="ties", T=256, d=256, E=32, num_local=32, k=6,
                                           F=256)
    pr = synth.make_problem(wl, seed=41)
    L = synth.tied_logits(wl.T, wl.E, levels=3, seed=42)
    gpu = forward(pr, logits_in=L)
    # many ties inside rows: the lower index must win every time
    assert torch.equal(gpu["logits"], L)
    check(pr, gpu, check_logits=False)


def test_non_finite_logits_route_as_the_oracle():
    """Rows holding NaN or +-inf route every slot to k distinct experts in
    [0, E), ordered as the oracle orders them (a NaN ranks as -inf; ties to the
    lower index), bit for bit; the finite rows are unaffected."""
    wl = synth.WORKLOADS["decode"].replace(name="nonfinite", T=96, d=256, E=32, num_local=32,
                                           k=4, F=256)
    pr = synth.make_problem(wl, seed=44)
    g = torch.Generator().manual_seed(45)
    L = torch.randn((wl.T, wl.E), generator=g)
    bad = [3, 17, 40, 41, 95]
    L[3, :] = float("nan")                      # all NaN: the k lowest ids
    L[17, 5] = float("nan")                     # one NaN: ranked last
    L[40, 7] = float("inf")                     # +inf: chosen first
    L[41, :] = float("-inf")
    L[95, ::2] = float("nan")
    gpu = forward(pr, logits_in=L)
    ids = gpu["topk_idx"].numpy()
    assert ((ids >= 0) & (ids < wl.E)).all()
    assert all(len(set(r.tolist())) == wl.k for r in ids)
    assert ids[3].tolist() == [0, 1, 2, 3] and ids[41].tolist() == [0, 1, 2, 3]
    assert 5 not in ids[17].tolist() and ids[40, 0] == 7
    assert all(i % 2 == 1 for i in ids[95].tolist())
    assert np.array_equal(ids, orc.topk_select(L.numpy(), wl.k)), "non-finite routing"
    # finite rows: routing and outputs as the oracle gives them (rows are
    # independent, so the non-finite rows are replaced by zeros there)
    good = np.array([t for t in range(wl.T) if t not in bad])
    Lz = L.clone()
    Lz[bad] = 0.0
    ref = oracle_for(pr, Lz, tokens=good)
    assert np.array_equal(ids[good], ref["topk_idx"][good])
    assert np.abs(gpu["topk_w"].numpy()[good] - ref["topk_w"][good]).max() <= 1e-6
    err = rel_l2(gpu["out"].float().numpy()[good], ref["out"])
    assert err <= TOL[(wl.act, wl.weight)]


def test_all_equal_logits_pick_the_lowest_experts():
    wl = synth.WORKLOADS["decode"].replace(name="flat", T=64, d=128, E=16, num_local=16, k=5, F=128)
    pr = synth.make_problem(wl, seed=43)
    gpu = forward(pr, logits_in=torch.zeros((64, 16)))
    assert torch.equal(gpu["topk_idx"], torch.arange(5, dtype=torch.int32).repeat(64, 1))
    assert torch.allclose(gpu["topk_w"], torch.full((64, 5), 0.2))


# Every token routed to the same k experts (planted logits, margin 10 over
# noise of 0.1), at sizes that select the prefill-sized tile plans: one or two
# experts then hold every slot (many M tiles of one expert, the others empty),
# the gate/up tail items are cut along K (d = 1024), and on an expert-parallel
# rank either two of the hot experts are local or none is (no local slot at
# all: both GEMMs get no item and every output row is 0).
HOT = {
    "bf16_wide_hot2": (synth.WORKLOADS["prefill"].replace(
        name="hot_bf16_T1500_d1024_E16_k2_F256", T=1500, d=1024, E=16, num_local=16, k=2, F=256,
        bias=(), seed=111), [3, 11]),
    "bf16_big_hot1": (synth.WORKLOADS["mixtral"].replace(
        name="hot_bf16_T2100_d512_E4_k1_F384", T=2100, d=512, E=4, num_local=4, k=1, F=384,
        bias=(), seed=112), [2]),
    "fp8_rank_hot": (synth.WORKLOADS["dsv3_rank"].replace(
        name="hot_fp8_T2000_d1024_E16_local0-7_k4_F384", T=2000, d=1024, E=16, num_local=8,
        expert_begin=0, k=4, F=384, bias=(), seed=113), [1, 5, 9, 13]),
    "fp8_rank_none_local": (synth.WORKLOADS["dsv3_rank"].replace(
        name="hot_fp8_T2000_d512_E16_local0-7_k4_F384_nonlocal", T=2000, d=512, E=16,
        num_local=8, expert_begin=0, k=4, F=384, bias=(), seed=114), [8, 9, 10, 11]),
    "mxfp4_hot": (synth.WORKLOADS["decode_mxfp4"].replace(
        name="hot_mxfp4_T2000_d1024_E16_k4_F384", T=2000, d=1024, E=16, num_local=16, k=4,
        F=384, bias=(), seed=115, regime="prefill"), [0, 6, 7, 15]),
}


@pytest.mark.parametrize("case", list(HOT))
def test_all_slots_on_the_same_experts(case):
    wl, hot = HOT[case]
    pr = synth.make_problem(wl)
    g = torch.Generator().manual_seed(wl.seed + 1)
    L = 0.1 * torch.randn((wl.T, wl.E), generator=g)
    L[:, hot] += 10.0
    gpu = forward(pr, logits_in=L)
    assert torch.equal(torch.sort(gpu["topk_idx"], dim=1).values,
                       torch.tensor(hot, dtype=torch.int32).repeat(wl.T, 1))
    ref, _ = check(pr, gpu, check_logits=False)
    local = [e for e in hot if wl.expert_begin <= e < wl.expert_begin + wl.num_local]
    assert int(ref["offsets"][-1]) == wl.T * len(local)
    if not local:
        assert torch.count_nonzero(gpu["out"]) == 0

def test_tokens_without_local_slot_get_zero_and_ranks_sum_to_the_layer():
    base = synth.WORKLOADS["dsv3_rank"].replace(name="ep4", T=128, d=256, E=16, k=2, F=256,
                                                expert_begin=0, num_local=16, weight="bf16")
    full = synth.make_problem(base, seed=51)
    g = upload(full)
    whole = forward(full, g)
    tot = torch.zeros_like(whole["out"], dtype=torch.float32)
    for r in range(4):
        wl = base.replace(expert_begin=4 * r, num_local=4)
        part = synth.Problem(wl, full.x, full.w_router, full.bias, full.w_gate[4 * r:4 * r + 4],
                             full.w_up[4 * r:4 * r + 4], full.w_down[4 * r:4 * r + 4])
        gp = forward(part)
        assert torch.equal(gp["topk_idx"], whole["topk_idx"])
        idx = gp["topk_idx"]
        none = ~((idx >= 4 * r) & (idx < 4 * r + 4)).any(1)
        assert torch.all(gp["out"][none] == 0)
        check(part, gp)
        tot += gp["out"].float()
    assert rel_l2(tot.numpy(), whole["out"].float().numpy()) <= 1e-2


def test_power_of_two_scaling_is_exact_and_runs_are_deterministic():
    wl = SMALL["bf16_skew"]
    pr = synth.make_problem(wl)
    g = upload(pr)
    a = forward(pr, g)
    b = forward(pr, g)
    for n in a:
        assert torch.equal(a[n], b[n]), n
    g2 = dict(g)
    g2["w_down"] = (g["w_down"].float() * 2).to(g["w_down"].dtype)
    c = forward(pr, g2)
    assert torch.equal((a["out"].float() * 2).to(a["out"].dtype), c["out"])


def test_standalone_calls_match_forward():
    wl = SMALL["fp8_rank_prefill"]
    pr = synth.make_problem(wl)
    g = upload(pr)
    ref = forward(pr, g)
    T, d, E, k, F, El = wl.T, wl.d, wl.E, wl.k, wl.F, wl.num_local
    p = _prob(wl)
    logits = torch.empty((T, E), dtype=torch.float32, device=DEV)
    idx = torch.empty((T, k), dtype=torch.int32, device=DEV)
    gw = torch.empty((T, k), dtype=torch.float32, device=DEV)
    B.moe_route(p, g["x"], g["w_router"], g["bias"], logits, idx, gw,
                B.workspace(p, B.MOE_CALL_ROUTE, DEV))
    counts = torch.empty((El,), dtype=torch.int32, device=DEV)
    offsets = torch.empty((El + 1,), dtype=torch.int32, device=DEV)
    ss = torch.empty((T * k,), dtype=torch.int32, device=DEV)
    sp = torch.empty((T * k,), dtype=torch.int32, device=DEV)
    B.moe_permute(p, idx, counts, offsets, ss, sp, B.workspace(p, B.MOE_CALL_PERMUTE, DEV))
    y = torch.empty((T * k, d), dtype=torch.bfloat16, device=DEV)
    B.moe_expert_ffn(p, g["x"], ss, offsets, g["w_gate"], g["w_up"], g["w_down"], g["s_gate"],
                     g["s_up"], g["s_down"], None, y, B.workspace(p, B.MOE_CALL_EXPERT_FFN, DEV))
    out = torch.empty((T, d), dtype=torch.bfloat16, device=DEV)
    B.moe_combine(p, y, sp, gw, out)   # gates applied in the combine this time
    torch.cuda.synchronize()
    assert torch.equal(idx.cpu(), ref["topk_idx"]) and torch.equal(offsets.cpu(), ref["offsets"])
    assert torch.equal(sp.cpu(), ref["slot_pos"])
    assert rel_l2(out.float().cpu().numpy(), ref["out"].float().numpy()) <= 1e-2


@pytest.mark.parametrize("T", [300, 3001])   # one-workgroup path, and the 3-kernel path
def test_permute_treats_out_of_range_ids_as_not_local(T):
    E, k, El = 16, 3, 16
    wl = synth.WORKLOADS["decode"].replace(T=T, d=128, E=E, num_local=El, k=k, F=128)
    p = _prob(wl)
    rng = np.random.default_rng(61)
    ids = rng.integers(-3, E + 3, size=(T, k)).astype(np.int32)
    ids[0, 0] = np.iinfo(np.int32).min
    ids[1, 0] = np.iinfo(np.int32).max
    idx = torch.from_numpy(ids).to(DEV)
    counts = torch.empty((El,), dtype=torch.int32, device=DEV)
    offsets = torch.empty((El + 1,), dtype=torch.int32, device=DEV)
    ss = torch.full((T * k,), -7, dtype=torch.int32, device=DEV)
    sp = torch.empty((T * k,), dtype=torch.int32, device=DEV)
    B.moe_permute(p, idx, counts, offsets, ss, sp, B.workspace(p, B.MOE_CALL_PERMUTE, DEV))
    torch.cuda.synchronize()
    c, o, s, q = orc.expert_permutation(ids, 0, El)
    assert np.array_equal(counts.cpu().numpy(), c) and np.array_equal(offsets.cpu().numpy(), o)
    assert np.array_equal(ss.cpu().numpy()[:o[-1]], s) and np.array_equal(sp.cpu().numpy(), q)


# ---------------------------------------------------------------- full sizes

def _sample(T, n, seed):
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(T, size=min(n, T), replace=False))


@pytest.mark.parametrize("layout,T", [("blocked", T) for T in (1, 2, 4, 8, 16, 64, 256, 1024, 4096)]
                         + [("rows", T) for T in (1, 2, 4, 8, 16, 64)])
def test_batch_sweep_parity(layout, T):
    """The Qwen3-shaped layer across the batch sizes of the sweep (the decode
    workload's distributions with T tokens): every tile plan from decode to
    prefill tiles (and the split-K gate/up path of the smallest batches), on
    a sample of tokens at the larger sizes; blocked weights as the sweep in
    bench.py runs them, and row-major ones at decode sizes (row-major prefill
    tiles are covered by the small cases)."""
    wl = synth.WORKLOADS["decode"].replace(name=f"qwen3_sweep_T{T}", T=T, seed=70 + T % 97)
    pr = synth.make_problem(wl)
    g = upload(pr)
    gpu = forward(pr, pack(pr, g), blocked=True) if layout == "blocked" else forward(pr, g)
    check(pr, gpu, tokens=None if T <= 64 else _sample(T, 24, seed=T))


@pytest.mark.parametrize("name,n_sample", [("decode", None), ("prefill", 96), ("mixtral", 32),
                                           ("dsv3_rank", 48), ("decode_mxfp4", None),
                                           ("prefill_mxfp4", 64)])
def test_full_size_workloads(name, n_sample):
    """Each workload at its full size in the configuration bench.py times
    (weights in the blocked layout), against the oracle; the row-major layout
    bit for bit where both sum the same K order, else against the oracle too."""
    wl = synth.WORKLOADS[name]
    print(f"generating {wl.name}", flush=True)
    pr = synth.make_problem(wl)
    g = upload(pr)
    gpu = forward(pr, pack(pr, g), blocked=True)
    tokens = None if n_sample is None else _sample(wl.T, n_sample, seed=7)
    ref, err = check(pr, gpu, tokens=tokens)
    rows = forward(pr, g)
    if same_plan_when_blocked(wl):
        for n in rows:
            assert torch.equal(rows[n], gpu[n]), n
    else:
        check(pr, rows, tokens=tokens)
    counts = ref["counts"]
    print(f"[{wl.name}] kept N={int(ref['offsets'][-1])} touched={int((counts > 0).sum())}/"
          f"{wl.num_local} max/mean={counts.max() / max(counts.mean(), 1e-9):.2f}", flush=True)
