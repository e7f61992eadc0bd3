"""The seeded input generator: determinism, distributions and formats."""
import json
import os

import numpy as np
import torch

from mixture_experts_layer_15_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_figures.json")


def _small(wl, **kw):
    return wl.replace(**kw)


def test_same_seed_same_bits_and_different_seed_differs():
    wl = _small(synth.WORKLOADS["decode"], T=16, E=8, num_local=8, d=256, F=128)
    a, b = synth.make_problem(wl), synth.make_problem(wl)
    c = synth.make_problem(wl, seed=99)
    for name in ("x", "w_router", "w_gate", "w_up", "w_down"):
        assert torch.equal(getattr(a, name), getattr(b, name))
        assert not torch.equal(getattr(a, name), getattr(c, name))


def test_shapes_formats_and_scales():
    wl = _small(synth.WORKLOADS["dsv3_rank"], T=32, d=256, F=384, E=16, num_local=4)
    p = synth.make_problem(wl)
    assert p.x.dtype == torch.bfloat16 and p.x.shape == (32, 256)
    assert p.w_router.shape == (256, 16) and p.bias.shape == (16,)
    assert p.w_gate.dtype == torch.uint8 and p.w_gate.shape == (4, 384, 256)
    assert p.w_down.shape == (4, 256, 384)
    assert p.s_gate.shape == (4, 3, 2) and p.s_down.shape == (4, 2, 3)
    # every 128x128 block uses its full range: |code| reaches 448 and no NaN code
    q = p.w_gate.view(torch.float8_e4m3fn).to(torch.float32)
    blocks = q.reshape(4, 3, 128, 2, 128).abs().amax(dim=(2, 4))
    assert torch.all(blocks == 448.0)
    assert not torch.isnan(q).any()


def test_distributions():
    wl = _small(synth.WORKLOADS["prefill"], T=512, d=512, F=256, E=8, num_local=8)
    p = synth.make_problem(wl)
    x = p.x.float()
    assert abs(x.mean().item()) < 0.01 and abs(x.std().item() - 1) < 0.01
    assert abs(p.w_gate.float().std().item() * np.sqrt(512) - 1) < 0.01
    assert abs(p.w_down.float().std().item() * np.sqrt(256) - 1) < 0.01
    e = np.arange(8)
    assert np.allclose(p.bias.numpy(), (2.0 * (e + 1.0) ** -1.1).astype(np.float32))


def test_workload_table_matches_the_pages_ep_block():
    g = json.load(open(GOLDEN))["ep_block"]
    wl = synth.WORKLOADS["dsv3_rank"]
    assert wl.E == g["routed_experts"] and wl.num_local == g["experts_per_gpu"]
    assert wl.E // wl.num_local == g["gpus"] and wl.F == g["intermediate"]
    r = json.load(open(GOLDEN))["routing_fanout"]
    assert (wl.E, wl.k) == (r["routed_experts"], r["selected_per_token"])


def test_raw_is_pure_reinterpretation():
    t = torch.tensor([1.0, -2.5, 3.0], dtype=torch.bfloat16)
    r = synth.raw(t)
    assert r.dtype == np.uint16
    assert np.array_equal((r.astype(np.uint32) << 16).view(np.float32), np.array([1.0, -2.5, 3.0], np.float32))
