"""moe_forward_noalloc (the whole layer with the library's own scratch array,
for callers that cannot allocate) against moe_forward with a caller
workspace: the same kernels, so the same bits, on two calls in a row, the
second with a smaller problem (the array keeps the first call's contents);
and against the oracle to the usual bar."""
import numpy as np
import pytest
import torch

from mixture_experts_layer_15_amd import binding as B
from mixture_experts_layer_15_amd import synth
from oracle import moe_oracle as orc

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load_library()


def _run(wl, noalloc):
    pr = synth.make_problem(wl)
    p = B.problem(wl.T, wl.d, wl.E, wl.k, wl.F, wl.expert_begin, wl.num_local, wl.act, wl.weight)
    g = {n: (None if getattr(pr, n) is None else getattr(pr, n).to(DEV))
         for n in ("x", "w_router", "bias", "w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down")}
    T, E, k, d, El = wl.T, wl.E, wl.k, wl.d, wl.num_local
    o = dict(out=torch.full((T, d), float("nan"), dtype=pr.x.dtype, device=DEV),
             logits=torch.empty((T, E), dtype=torch.float32, device=DEV),
             topk_idx=torch.empty((T, k), dtype=torch.int32, device=DEV),
             topk_w=torch.empty((T, k), dtype=torch.float32, device=DEV),
             counts=torch.empty((El,), dtype=torch.int32, device=DEV),
             offsets=torch.empty((El + 1,), dtype=torch.int32, device=DEV),
             sorted_slot=torch.empty((T * k,), dtype=torch.int32, device=DEV),
             slot_pos=torch.empty((T * k,), dtype=torch.int32, device=DEV))
    kw = dict(x=g["x"], w_router=g["w_router"], router_bias=g["bias"], w_gate=g["w_gate"],
              w_up=g["w_up"], w_down=g["w_down"], s_gate=g["s_gate"], s_up=g["s_up"],
              s_down=g["s_down"], **o)
    if noalloc:
        assert B.moe_workspace_size(p, B.MOE_CALL_FORWARD) <= B.MOE_NOALLOC_SCRATCH_BYTES
        B.moe_forward_noalloc(p, **kw)
    else:
        B.moe_forward(p, ws=B.workspace(p, B.MOE_CALL_FORWARD, DEV), **kw)
    torch.cuda.synchronize()
    return pr, {n: t.cpu() for n, t in o.items()}


CALLS = [
    # the Qwen3-30B-A3B decode step, then a smaller batch of another shape with
    # a skewed router, on an expert-parallel block with FP8 weights
    synth.WORKLOADS["decode"],
    synth.WORKLOADS["dsv3_rank"].replace(name="noalloc_fp8_T40_d512_E32_local8-23_k4_F256",
                                         T=40, d=512, E=32, num_local=16, expert_begin=8, k=4,
                                         F=256, seed=91),
]


def test_noalloc_forward_matches_workspace_forward_on_two_calls():
    for wl in CALLS:
        print(f"[noalloc] {wl.name}", flush=True)
        pr, got = _run(wl, noalloc=True)
        _, ref = _run(wl, noalloc=False)
        N = int(ref["offsets"][-1])
        for n in got:
            a, b = got[n], ref[n]
            if n == "sorted_slot":   # rows past N are unspecified
                a, b = a[:N], b[:N]
            assert torch.equal(a, b), (wl.name, n)
        # and the oracle's bar: routing bit-exact, output within tolerance
        o = orc.moe_layer_forward(synth.raw(pr.x), got["logits"].numpy(), wl.k,
                                  synth.raw(pr.w_gate), synth.raw(pr.w_up), synth.raw(pr.w_down),
                                  act_fmt=wl.act, weight_fmt=wl.weight, e0=wl.expert_begin,
                                  E_l=wl.num_local, s_gate=synth.raw(pr.s_gate),
                                  s_up=synth.raw(pr.s_up), s_down=synth.raw(pr.s_down))
        assert np.array_equal(got["topk_idx"].numpy(), o["topk_idx"])
        assert np.array_equal(got["slot_pos"].numpy(), o["slot_pos"])
        out = got["out"].float().numpy().astype(np.float64)
        err = np.linalg.norm(out - o["out"]) / np.linalg.norm(o["out"])
        print(f"[noalloc] {wl.name}: bits equal to moe_forward, rel L2 {err:.3e}", flush=True)
        assert err <= 1e-2
