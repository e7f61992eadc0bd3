"""Seeded synthetic inputs for the MoE layer, and the workload table.

This module only draws numbers and stores them in the formats the layer
consumes (float32, bfloat16, or FP8 E4M3FN codes with 128x128 block scales).
It holds none of the layer's arithmetic: the library and the CPU checker both
receive what it produces and nothing else.

No dataset or trained checkpoint is used.  The workloads stand in for the
traffic classes named in the benchmark plan of "Развертывание vLLM Expert
Parallel для DeepSeek и других моделей MoE" (flatkey.ai), section on the
benchmarking plan: short-prompt high-concurrency decode, long-prompt prefill,
and an expert-skewed trace; the model shapes are those the pages discuss
(Qwen3-30B-A3B, Mixtral-8x7B, DeepSeek-V3).

Draw order for a given seed (``numpy.random.default_rng``, PCG64): ``x``,
``W_r``, the router bias (when drawn), then for each local expert in id order
``w_gate``, ``w_up``, ``w_down``.  Every matrix is drawn float32 as
``N(0, 1) / sqrt(fan_in)`` directly in its stored "out x in" orientation
(fan_in = d for router, gate and up; F for down) and then rounded to
nearest-even into the storage format.  FP8 weights use per-128x128-block
scales ``s = amax(block) / 448`` (``s = 1`` for an all-zero block) and codes
``RNE(W / s)`` clamped to +-448.  MXFP4 weights use, per 32 consecutive "in"
values of a row, the shared exponent ``X = floor(log2(amax)) - 2`` (the OCP MX
recipe: 2 is E2M1's largest exponent; ``X = 0`` for an all-zero block) stored
as the E8M0 byte ``X + 127`` (clamped to 0..252), and codes = ``W / 2^X``
rounded to the nearest E2M1 value (ties to the smaller magnitude), clamped
to +-6.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

FP8_MAX = 448.0
BLOCK = 128
MX_BLOCK = 32
# E2M1 magnitudes of codes 0..7 and the midpoints between neighbours
_E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
_E2M1_MID = (_E2M1[1:] + _E2M1[:-1]) / 2


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    E: int
    k: int
    F: int
    expert_begin: int
    num_local: int
    act: str            # "f32" | "bf16"
    weight: str         # "f32" | "bf16" | "fp8" | "mxfp4"
    bias: tuple = ()    # () | ("zipf", s, scale) | ("gauss", sd)
    seed: int = 0
    regime: str = "prefill"   # "decode" (HBM-bound) | "prefill" (MFMA-bound) | "tiny"

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads (shapes, formats and router skew of the pages' models).
WORKLOADS = {
    "tiny": Workload("tiny_fp32_T64_d128_E8_k2_F256", T=64, d=128, E=8, k=2, F=256,
                     expert_begin=0, num_local=8, act="f32", weight="f32", seed=1, regime="tiny"),
    "decode": Workload("qwen3_30b_a3b_decode_T64_d2048_E128_k8_F768", T=64, d=2048, E=128, k=8,
                       F=768, expert_begin=0, num_local=128, act="bf16", weight="bf16", seed=2,
                       regime="decode"),
    "prefill": Workload("qwen3_30b_a3b_prefill_T8192_d2048_E128_k8_F768_zipf1.1", T=8192, d=2048,
                        E=128, k=8, F=768, expert_begin=0, num_local=128, act="bf16", weight="bf16",
                        bias=("zipf", 1.1, 2.0), seed=3),
    "mixtral": Workload("mixtral_8x7b_T4096_d4096_E8_k2_F14336_gauss1.0", T=4096, d=4096, E=8, k=2,
                        F=14336, expert_begin=0, num_local=8, act="bf16", weight="bf16",
                        bias=("gauss", 1.0), seed=4),
    "decode_mxfp4": Workload("qwen3_30b_a3b_decode_T64_d2048_E128_k8_F768_mxfp4", T=64, d=2048,
                             E=128, k=8, F=768, expert_begin=0, num_local=128, act="bf16",
                             weight="mxfp4", seed=6, regime="decode"),
    "prefill_mxfp4": Workload("qwen3_30b_a3b_prefill_T8192_d2048_E128_k8_F768_zipf1.1_mxfp4",
                              T=8192, d=2048, E=128, k=8, F=768, expert_begin=0, num_local=128,
                              act="bf16", weight="mxfp4", bias=("zipf", 1.1, 2.0), seed=7),
    "dsv3_rank": Workload("deepseek_v3_ep_rank_T16384_d7168_E256_local0-31_k8_F2048_fp8_zipf1.2",
                          T=16384, d=7168, E=256, k=8, F=2048, expert_begin=0, num_local=32,
                          act="bf16", weight="fp8", bias=("zipf", 1.2, 2.0), seed=5),
    # Two sensitivity rows, reported beside the gated ones.  The prefill with
    # the Zipf bias scaled to 1.0 instead of 2.0 (same seed, so the same
    # tokens and weights): a max/mean expert load of about 4, inside the
    # "3-5x" the prefill workload's text states, which its own 2.0 recipe
    # overshoots.  The DeepSeek-V3 rank at T = 4096 without a bias: about 4096
    # kept slots, the count the rank workload's text states, which its own
    # T = 16384 recipe exceeds seven times; about 128 rows per expert, so the
    # expert GEMMs sit near the HBM roofline there.
    "prefill_cal": Workload("qwen3_30b_a3b_prefill_T8192_d2048_E128_k8_F768_zipf1.1x1.0",
                            T=8192, d=2048, E=128, k=8, F=768, expert_begin=0, num_local=128,
                            act="bf16", weight="bf16", bias=("zipf", 1.1, 1.0), seed=3),
    "dsv3_rank_4k": Workload("deepseek_v3_ep_rank_T4096_d7168_E256_local0-31_k8_F2048_fp8",
                             T=4096, d=7168, E=256, k=8, F=2048, expert_begin=0, num_local=32,
                             act="bf16", weight="fp8", seed=8),
}


@dataclasses.dataclass
class Problem:
    """One seeded instance, all tensors on the CPU in storage format."""
    wl: Workload
    x: torch.Tensor                   # [T, d] float32 | bfloat16
    w_router: torch.Tensor            # [d, E] same dtype as x
    bias: Optional[torch.Tensor]      # [E] float32 or None
    w_gate: torch.Tensor              # [E_l, F, d] float32 | bfloat16 | uint8 (fp8 codes);
                                      # mxfp4: [E_l, F, d/2] uint8, two codes per byte
    w_up: torch.Tensor                # [E_l, F, d]
    w_down: torch.Tensor              # [E_l, d, F]
    s_gate: Optional[torch.Tensor] = None   # fp8: [E_l, F/128, d/128] float32;
                                            # mxfp4: [E_l, d/32, F] uint8 E8M0
    s_up: Optional[torch.Tensor] = None
    s_down: Optional[torch.Tensor] = None   # [E_l, d/128, F/128]


def _act_dtype(fmt: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[fmt]


def _store(a32: np.ndarray, fmt: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32))
    if fmt == "f32":
        return t.clone()
    if fmt == "bf16":
        return t.to(torch.bfloat16)
    raise ValueError(fmt)


def quantize_fp8_block128(w32: np.ndarray):
    """float32 [R, C] -> (uint8 E4M3FN codes [R, C], float32 scales [R/128, C/128])."""
    R, C = w32.shape
    assert R % BLOCK == 0 and C % BLOCK == 0
    t = torch.from_numpy(np.ascontiguousarray(w32, dtype=np.float32))
    blocks = t.reshape(R // BLOCK, BLOCK, C // BLOCK, BLOCK)
    amax = blocks.abs().amax(dim=(1, 3))
    s = amax / FP8_MAX
    s = torch.where(amax == 0, torch.ones_like(s), s)
    scaled = (blocks / s[:, None, :, None]).clamp(-FP8_MAX, FP8_MAX)
    q = scaled.reshape(R, C).to(torch.float8_e4m3fn).view(torch.uint8)
    return q.contiguous(), s.contiguous()


def quantize_mxfp4(w32: np.ndarray):
    """float32 [R, C] -> (uint8 codes [R, C/2], two per byte, element 2j in
    the low nibble of byte j; uint8 E8M0 scales [C/32, R], block-major)."""
    R, C = w32.shape
    assert C % MX_BLOCK == 0
    blocks = np.asarray(w32, dtype=np.float64).reshape(R, C // MX_BLOCK, MX_BLOCK)
    amax = np.abs(blocks).max(axis=2)
    with np.errstate(divide="ignore"):
        X = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2, 0.0)
    sbyte = np.clip(X + 127, 0, 252).astype(np.int64)
    v = blocks / np.exp2(sbyte - 127)[:, :, None]
    mag = np.searchsorted(_E2M1_MID, np.abs(v), side="left")  # ties -> smaller magnitude
    codes = (mag | np.where(v < 0, 8, 0)).astype(np.uint8).reshape(R, C)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return torch.from_numpy(packed), torch.from_numpy(np.ascontiguousarray(sbyte.T.astype(np.uint8)))


def router_bias(wl: Workload, rng: np.random.Generator) -> Optional[np.ndarray]:
    """Per-expert logit bias that skews the expert load.

    ``("zipf", s, scale)``: ``b_e = scale * (e + 1)^-s`` (expert id order is the
    Zipf rank order).  ``("gauss", sd)``: ``b_e ~ N(0, sd^2)`` drawn after ``W_r``.
    """
    if not wl.bias:
        return None
    kind = wl.bias[0]
    if kind == "zipf":
        _, s, scale = wl.bias
        e = np.arange(wl.E, dtype=np.float64)
        return (scale * (e + 1.0) ** (-s)).astype(np.float32)
    if kind == "gauss":
        sd = wl.bias[1]
        return (rng.standard_normal(wl.E, dtype=np.float32) * np.float32(sd)).astype(np.float32)
    raise ValueError(kind)


def make_problem(wl: Workload, seed: Optional[int] = None) -> Problem:
    """Draw one instance of ``wl`` (see the module docstring for the recipe)."""
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    T, d, E, F, El = wl.T, wl.d, wl.E, wl.F, wl.num_local
    x = _store(rng.standard_normal((T, d), dtype=np.float32), wl.act)
    w_r = _store(rng.standard_normal((d, E), dtype=np.float32) * np.float32(1.0 / math.sqrt(d)), wl.act)
    b = router_bias(wl, rng)
    bias = None if b is None else torch.from_numpy(b)

    wfmt = wl.weight
    gdt = torch.uint8 if wfmt in ("fp8", "mxfp4") else _act_dtype(wfmt)
    div = 2 if wfmt == "mxfp4" else 1   # two 4-bit codes per byte along "in"
    w_gate = torch.empty((El, F, d // div), dtype=gdt)
    w_up = torch.empty((El, F, d // div), dtype=gdt)
    w_down = torch.empty((El, d, F // div), dtype=gdt)
    s_gate = s_up = s_down = None
    if wfmt == "fp8":
        s_gate = torch.empty((El, F // BLOCK, d // BLOCK), dtype=torch.float32)
        s_up = torch.empty_like(s_gate)
        s_down = torch.empty((El, d // BLOCK, F // BLOCK), dtype=torch.float32)
    if wfmt == "mxfp4":
        s_gate = torch.empty((El, d // MX_BLOCK, F), dtype=torch.uint8)
        s_up = torch.empty_like(s_gate)
        s_down = torch.empty((El, F // MX_BLOCK, d), dtype=torch.uint8)
    gd, gf = np.float32(1.0 / math.sqrt(d)), np.float32(1.0 / math.sqrt(F))
    for j in range(El):
        g = rng.standard_normal((F, d), dtype=np.float32) * gd
        u = rng.standard_normal((F, d), dtype=np.float32) * gd
        dn = rng.standard_normal((d, F), dtype=np.float32) * gf
        if wfmt == "fp8":
            w_gate[j], s_gate[j] = quantize_fp8_block128(g)
            w_up[j], s_up[j] = quantize_fp8_block128(u)
            w_down[j], s_down[j] = quantize_fp8_block128(dn)
        elif wfmt == "mxfp4":
            w_gate[j], s_gate[j] = quantize_mxfp4(g)
            w_up[j], s_up[j] = quantize_mxfp4(u)
            w_down[j], s_down[j] = quantize_mxfp4(dn)
        else:
            w_gate[j] = _store(g, wfmt)
            w_up[j] = _store(u, wfmt)
            w_down[j] = _store(dn, wfmt)
    return Problem(wl, x, w_r, bias, w_gate, w_up, w_down, s_gate, s_up, s_down)


def tokens(wl: Workload, seed: int) -> torch.Tensor:
    """Another batch of ``wl.T`` tokens, ``x ~ N(0, 1)`` in the activation
    format, from its own seed (the router and experts stay those of
    ``make_problem``): a second sample of the same traffic."""
    rng = np.random.default_rng(seed)
    return _store(rng.standard_normal((wl.T, wl.d), dtype=np.float32), wl.act)


def tied_logits(T: int, E: int, levels: int, seed: int) -> torch.Tensor:
    """float32 logits ``[T, E]`` drawn from only ``levels`` distinct values, so
    that ties inside a row are frequent (for checking the lower-index rule)."""
    rng = np.random.default_rng(seed)
    vals = rng.integers(0, levels, size=(T, E)).astype(np.float32) * np.float32(0.25)
    return torch.from_numpy(vals)


def raw(t: Optional[torch.Tensor]) -> Optional[np.ndarray]:
    """Storage bits as numpy: float32 as is, bfloat16 as uint16 patterns,
    FP8 codes as uint8.  Pure reinterpretation, no arithmetic."""
    if t is None:
        return None
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    return t.numpy()
