"""Benchmark of the MoE layer forward on one MI355X.

One step = one ``moe_forward`` call (router, top-k gating, permutation, both
expert GEMMs, combine) over one batch of synthetic tokens already resident in
HBM.  The default workload is the Qwen3-30B-A3B-shaped decode step (T=64,
d=2048, E=128, k=8, F=768, bf16), which streams most expert weights from HBM
("Serve MoE models with expert parallelism", section "Start with one device if
the model fits": a batch of many tokens touches many experts, so a decode step
reads more of the weights as the batch grows).  ``--config`` selects the other
workloads (prefill, mixtral, dsv3_rank, tiny).

Weights are held in several copies in HBM and the steps rotate through them,
so that no step finds another step's weights in the 256 MB Infinity Cache.

Prints one JSON line: whole-layer tokens/s, plus a roofline object for the
dominant kernel (the gate/up grouped GEMM) timed with HIP events on the
library's stream, and a CPU baseline of the float64 oracle on a bounded sample.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from mixture_experts_layer_15_amd import binding as B  # noqa: E402
from mixture_experts_layer_15_amd import synth  # noqa: E402

METRIC = "MoE-layer tokens/s; % of MFMA peak (prefill) or HBM GB/s peak (decode)"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, GB/s
PEAK_BF16_TFLOPS = 2500.0      # dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0       # dense fp8 MFMA
PEAK_FP32_TFLOPS = 157.3       # fp32 vector / matrix
ACT_BYTES = {"f32": 4, "bf16": 2}
W_BYTES = {"f32": 4, "bf16": 2, "fp8": 1, "mxfp4": 0.5}
W_BITS = {"f32": 32, "bf16": 16, "fp8": 8, "mxfp4": 4}



def gate_up_kernel_name(wl: synth.Workload, blocked: bool = False) -> str:
    """The gate/up kernel the library launches for this workload, as a
    rocprofv3 kernel trace names it (the library's tile plan: 32-row decode
    tiles up to 16 slots per expert on average, 64-row ones up to 64 (FP8: the
    32-row ones; MXFP4: the wave-streamed kernel on blocked weights, 32-row
    tiles with 128-deep steps on row-major ones), then 128 x 512 tiles for FP8
    and MXFP4, 256 x 256 from 512 slots per expert, else 128 x 512)."""
    S, El = wl.T * wl.k, wl.num_local
    if wl.weight == "f32":
        return "grouped_f32_kernel<true>"
    bits = W_BITS[wl.weight]
    if wl.weight == "mxfp4":
        if S <= 64 * El:
            if blocked:
                return "stream_gemm_kernel<true, 4, 4, 2, 2>"
            return "grouped_gemm_kernel<1, 1, 2, 4, true, 4, 128, 2, 3, false, false>"
        args = "4, 1, 2, 8, true, 4, 64, 4, 1"
    elif S <= 16 * El or (S <= 64 * El and wl.weight == "fp8"):
        args = f"1, 1, 2, 4, true, {bits}, 64, 4, {2 if wl.weight == 'fp8' else 1}"
    elif S <= 64 * El:
        args = "2, 1, 2, 4, true, 16, 64, 4, 1"
    elif wl.weight == "fp8":
        args = "4, 1, 2, 8, true, 8, 64, 2, 1"
    elif S >= 512 * El:
        args = "2, 4, 4, 2, true, 16, 64, 2, 1"
    else:
        args = "2, 2, 4, 4, true, 16, 64, 2, 1"
    return f"grouped_gemm_kernel<{args}, false, {'true' if blocked else 'false'}>"


def expert_bytes(d: int, F: int, wfmt: str, n_experts: int, with_scales: bool = True) -> int:
    """Weight bytes of n whole SwiGLU experts: 3 d F parameters each, times the
    bytes per parameter ("Expert Parallelism for MoE Models", section "Memory
    Sizing Equations": expert memory = experts x parameters per expert x bytes
    per parameter), plus the FP8 block scales."""
    b = int(n_experts * 3 * d * F * W_BYTES[wfmt])
    if wfmt == "fp8" and with_scales:
        b += n_experts * 3 * (d // 128) * (F // 128) * 4
    if wfmt == "mxfp4" and with_scales:
        b += n_experts * 3 * (d * F // 32)          # one E8M0 byte per 32 weights
    return b


def algorithmic(wl: synth.Workload, counts: np.ndarray, tokens_read: int) -> dict:
    """Algorithmic FLOPs and HBM bytes of one layer step and of the gate/up GEMM:
    the touched local experts' weights (and FP8 scales) once, the router matrix
    (when routing is part of the share), the token rows that have a local slot
    once, and the output once; FLOPs 2 T d E (router) + 6 N d F."""
    d, F, E, T, k = wl.d, wl.F, wl.E, wl.T, wl.k
    ab, wb = ACT_BYTES[wl.act], W_BYTES[wl.weight]
    N = int(counts.sum())
    touched = int((counts > 0).sum())
    router_flop = 2 * T * d * E
    router_bytes = d * E * ab
    expert_flop = 6 * N * d * F
    expert_bytes_ = expert_bytes(d, F, wl.weight, touched) + tokens_read * d * ab + T * d * ab
    gu_flop = 4 * N * d * F
    gu_scales = (2 * (d // 128) * (F // 128) * 4 if wl.weight == "fp8"
                 else 2 * d * F // 32 if wl.weight == "mxfp4" else 0)
    # the method's bytes: the touched experts' gate and up weights (and
    # scales) and the token rows read once; the materialised h is the
    # implementation's traffic, reported beside it
    gu_bytes = int(touched * (2 * d * F * wb + gu_scales) + tokens_read * d * ab)
    dn_flop = 2 * N * F * d
    dn_bytes = int(touched * (d * F * wb + gu_scales // 2))
    return dict(N=N, touched=touched, tokens_read=tokens_read,
                layer_flop=router_flop + expert_flop, layer_bytes=router_bytes + expert_bytes_,
                expert_flop=expert_flop, expert_bytes=expert_bytes_,
                gu_flop=gu_flop, gu_bytes=gu_bytes, gu_bytes_with_h=gu_bytes + N * F * ab,
                dn_flop=dn_flop, dn_bytes=dn_bytes,
                gu_unit_bytes=int(2 * d * F * wb + gu_scales))


class HipEvents:
    """Raw hipEvent_t handles (for the events moe_forward records on its stream)."""

    def __init__(self, n: int):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.arr = (ctypes.c_void_p * n)()
        for i in range(n):
            h = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(h)) == 0
            self.arr[i] = h.value

    def sync(self, i: int) -> None:
        assert self.hip.hipEventSynchronize(ctypes.c_void_p(self.arr[i])) == 0

    def ms(self, a: int, b: int) -> float:
        out = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(out), ctypes.c_void_p(self.arr[a]),
                                            ctypes.c_void_p(self.arr[b])) == 0
        return float(out.value)


def gemm_sources_sha256() -> str:
    """Hash of the expert-GEMM sources (the kernels a traffic record covers)."""
    import hashlib
    m = hashlib.sha256()
    for f in GEMM_SOURCES:
        m.update(open(os.path.join(ROOT, f), "rb").read())
    return m.hexdigest()


GEMM_SOURCES = ["mixture_experts_layer_15_amd/csrc/ffn.hip",
                "mixture_experts_layer_15_amd/csrc/moe_device.h",
                "mixture_experts_layer_15_amd/csrc/moe_internal.h"]


def measured_traffic(workload: str, kernel: str, layout: str):
    """HBM bytes per dispatch of `kernel` from the committed rocprofv3
    FETCH_SIZE/WRITE_SIZE runs (scaled by the copy-kernel calibration), or None
    when no record covers this workload and kernel or the record was taken on
    other kernel sources (each record carries the hash of the sources it was
    measured on)."""
    path = os.path.join(ROOT, "profiles", "gate_up_pmc.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    now = gemm_sources_sha256()
    for r in rec["records"]:
        if (r["workload"] == workload and r["kernel"] == kernel
                and r.get("weight_layout", "rows") == layout and r.get("source_sha256") == now):
            return int(r["traffic_bytes_per_dispatch"])
    return None


def cpu_baseline(pr: synth.Problem, logits: torch.Tensor, budget_s: float,
                 n_sample: int = 64) -> dict:
    """The float64 oracle, as it stands, on whole steps of the same workload
    (or on a sample of n_sample tokens when one step would exceed the budget;
    at least one repetition whatever the budget)."""
    from oracle import moe_oracle as orc
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    wl = pr.wl
    raw = {n: synth.raw(getattr(pr, n)) for n in ("x", "w_router", "w_gate", "w_up", "w_down",
                                                  "s_gate", "s_up", "s_down")}
    bias = None if pr.bias is None else pr.bias.numpy()
    L32 = logits.cpu().numpy()
    rng = np.random.default_rng(0)
    # a sample small enough for ~budget_s of work: whole steps when cheap
    sample = None if wl.T <= 256 else np.sort(rng.choice(wl.T, size=n_sample, replace=False))
    n_tok, t0, reps = 0, time.perf_counter(), 0
    while True:
        x64 = orc.decode_act(raw["x"] if sample is None else raw["x"][sample], wl.act)
        orc.router_logits(x64, orc.decode_act(raw["w_router"], wl.act), bias)
        orc.moe_layer_forward(raw["x"], L32, wl.k, raw["w_gate"], raw["w_up"], raw["w_down"],
                              act_fmt=wl.act, weight_fmt=wl.weight, e0=wl.expert_begin,
                              E_l=wl.num_local, s_gate=raw["s_gate"], s_up=raw["s_up"],
                              s_down=raw["s_down"], tokens=sample)
        n_tok += wl.T if sample is None else len(sample)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 50:
            break
    what = (f"{reps} whole step(s) of T={wl.T}" if sample is None else
            f"{reps} x {n_sample} sampled tokens of T={wl.T} (routing of all T each time)")
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:  # pragma: no cover
        pass
    return {"value": n_tok / el, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": what, "seconds": round(el, 2),
            "host_cpus": len(os.sched_getaffinity(0)), "cpu_model": model,
            "blas_threads": int(threads)}


def measure(wl: synth.Workload, steps: int, warmup: int, copies: int, dev,
            blocked: bool = False, warm: bool = True) -> dict:
    """Time `steps` moe_forward calls (after `warmup`) rotating `copies` weight
    copies, then the same steps with the library's stage events, then a warm
    pass on one copy.  Returns times and the routing statistics.  blocked:
    the weights are converted once (untimed, like a load-time conversion) to
    the library's blocked layout."""
    pr = synth.make_problem(wl)
    p = B.problem(wl.T, wl.d, wl.E, wl.k, wl.F, wl.expert_begin, wl.num_local, wl.act, wl.weight,
                  blocked=blocked)
    x = pr.x.to(dev)
    wr = pr.w_router.to(dev)
    bias = None if pr.bias is None else pr.bias.to(dev)
    wsets = []
    for c in range(copies):
        ws_ = {n: (None if getattr(pr, n) is None else getattr(pr, n).to(dev))
               for n in ("w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down")}
        if blocked:
            for n, which in (("w_gate", 0), ("w_up", 0), ("w_down", 1)):
                dst = torch.empty_like(ws_[n])
                B.moe_pack_weights(p, which, ws_[n], dst)
                ws_[n] = dst
            torch.cuda.synchronize()
        wsets.append(ws_)
    out = torch.empty((wl.T, wl.d), dtype=pr.x.dtype, device=dev)
    logits = torch.empty((wl.T, wl.E), dtype=torch.float32, device=dev)
    counts = torch.empty((wl.num_local,), dtype=torch.int32, device=dev)
    slot_pos = torch.empty((wl.T * wl.k,), dtype=torch.int32, device=dev)
    ws = B.workspace(p, B.MOE_CALL_FORWARD, dev)
    stream = torch.cuda.current_stream()

    def step(i: int, events=None) -> None:
        w = wsets[i % copies]
        B.moe_forward(p, x=x, w_router=wr, router_bias=bias, w_gate=w["w_gate"], w_up=w["w_up"],
                      w_down=w["w_down"], s_gate=w["s_gate"], s_up=w["s_up"], s_down=w["s_down"],
                      out=out, ws=ws, logits=logits, counts=counts, slot_pos=slot_pos,
                      events=events, stream=stream)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    print(f"[bench] {wl.name}: warmup {warmup} done, timing {steps} steps ({copies} weight "
          "copies)", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / steps

    # Stage times: the same steps again, with HIP events recorded by the library
    # on its stream at every stage boundary.
    ev_sets = [HipEvents(B.MOE_FORWARD_EVENTS) for _ in range(steps)]
    for i in range(steps):
        step(i, ev_sets[i].arr)
    torch.cuda.synchronize()
    names = ["route", "permute", "schedule", "gate_up", "down", "combine"]
    stage = {n: [] for n in names}
    layer_ev = []
    for e in ev_sets:
        e.sync(6)
        for s_i, n in enumerate(names):
            stage[n].append(e.ms(s_i, s_i + 1))
        layer_ev.append(e.ms(0, 6))
    stage_ms = {n: float(np.mean(v)) for n, v in stage.items()}
    share_ev = [l - r for l, r in zip(layer_ev, stage["route"])]  # permute .. combine

    # warm: one weight copy, so that the Infinity Cache may serve part of it (info)
    warm_ms = None
    if warm:
        warm_steps = max(steps // 2, 5)
        for i in range(3):
            step(0)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(warm_steps):
            step(0)
        torch.cuda.synchronize()
        warm_ms = (time.perf_counter() - t0) * 1e3 / warm_steps

    sp = slot_pos.cpu().numpy().reshape(wl.T, wl.k)
    tokens_read = int((sp >= 0).any(axis=1).sum())
    return dict(pr=pr, logits=logits, counts=counts.cpu().numpy(), tokens_read=tokens_read,
                ms_per_step=ms_per_step, stage_ms=stage_ms, stage_ev=stage, layer_ev=layer_ev,
                share_ev=share_ev, warm_ms=warm_ms, copies=copies)


# Dense bf16 GEMMs with the FLOPs of the prefill workloads' expert GEMMs
# (rows = kept slots, all experts' rows against one weight matrix): what the
# vendor library reaches on the same shapes without the gather, the ragged
# expert segments or the SwiGLU epilogue.  (name, rows M, output columns N,
# reduction K)
DENSE_REF = [("qwen3_prefill_gate_up", 65536, 1536, 2048), ("qwen3_prefill_down", 65536, 2048, 768),
             ("mixtral_gate_up", 8192, 28672, 4096), ("mixtral_down", 8192, 4096, 14336),
             ("dsv3_rank_gate_up", 28535, 4096, 7168), ("dsv3_rank_down", 28535, 7168, 2048)]


def dense_ref(args, dev) -> None:
    """torch.matmul on [M, K] x [K, N] bf16 (both operands contiguous), timed
    with events on the current stream: one JSON line per GEMM."""
    g = torch.Generator(device="cpu").manual_seed(0)
    for name, M, N, K in DENSE_REF:
        a = torch.randn((M, K), generator=g).to(torch.bfloat16).to(dev)
        b = (torch.randn((K, N), generator=g) / K ** 0.5).to(torch.bfloat16).to(dev)
        for _ in range(5):
            c = torch.matmul(a, b)
        torch.cuda.synchronize()
        n = args.steps or 20
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            c = torch.matmul(a, b)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / n
        tflops = 2.0 * M * N * K / (ms * 1e-3) / 1e12
        print(json.dumps({"dense_ref": name, "M": M, "N": N, "K": K, "ms": round(ms, 4),
                          "tflops": round(tflops, 1), "frac_mfma_bf16": round(tflops / 2500.0, 4),
                          "library": "torch.matmul (hipBLASLt)"}), flush=True)
        del a, b, c
        torch.cuda.empty_cache()


def pct(v, q) -> float:
    return round(float(np.percentile(np.asarray(v), q)), 5)


def sweep(args, dev) -> None:
    """Batch sweep at the Qwen3-30B-A3B shape: as T grows, the experts touched
    (hence the weight bytes) saturate while the FLOPs keep growing, and the
    layer moves from the HBM roofline to the MFMA one.  One JSON line per T."""
    base = synth.WORKLOADS["decode"]
    for T in [int(t) for t in args.sweep.split(",")]:
        wl = base.replace(name=f"qwen3_30b_a3b_T{T}_d2048_E128_k8_F768", T=T)
        steps = args.steps or (100 if T <= 512 else 20)
        m = measure(wl, steps, args.warmup if args.warmup is not None else 5, 4, dev,
                    args.layout == "blocked")
        alg = algorithmic(wl, m["counts"], m["tokens_read"])
        t = m["ms_per_step"] * 1e-3
        gu = m["stage_ms"]["gate_up"] * 1e-3
        print(json.dumps({
            "sweep": "qwen3_30b_a3b_batch", "T": T, "weight_layout": args.layout,
            "touched_experts": alg["touched"],
            "kept_slots": alg["N"], "ms_per_step": round(m["ms_per_step"], 5),
            "tokens_per_s": round(T / t, 1),
            "layer": {"alg_bytes": alg["layer_bytes"], "alg_flop": alg["layer_flop"],
                      "gbs": round(alg["layer_bytes"] / t / 1e9, 1),
                      "frac_hbm": round(alg["layer_bytes"] / t / 1e9 / PEAK_HBM_GBS, 4),
                      "tflops": round(alg["layer_flop"] / t / 1e12, 2),
                      "frac_mfma_bf16": round(alg["layer_flop"] / t / 1e12 / PEAK_BF16_TFLOPS, 4),
                      "flop_per_byte": round(alg["layer_flop"] / alg["layer_bytes"], 1)},
            "gate_up": {"ms": round(m["stage_ms"]["gate_up"], 5),
                        "gbs": round(alg["gu_bytes"] / gu / 1e9, 1),
                        "tflops": round(alg["gu_flop"] / gu / 1e12, 2)},
            "stage_ms": {n: round(v, 5) for n, v in m["stage_ms"].items()},
        }), flush=True)


def eplb(args, dev) -> None:
    """Expert-parallel load balancing at the DeepSeek-V3 shape (T = 16384,
    d = 7168, E = 256, k = 8, F = 2048, FP8 weights, Zipf-skewed router) on
    G = 8 ranks ("Serving MoE models with expert parallelism on 8xH200",
    section "Routing imbalance": copies of hot experts on less-loaded GPUs).

    The plan is made from the per-expert counts of one batch (the window) and
    measured on another batch of the same traffic.  Every rank's share
    (dispatch, expert FFN on its physical slots, combine) runs on this GPU,
    one rank after another, timed with events on the library's stream; with
    the ranks running side by side the layer waits for the slowest one.  The
    rank weights are random experts of the workload's shape (the kernels'
    time does not depend on their values; the copies' parity is tested
    separately).  One JSON line per placement."""
    G = 8
    base = synth.WORKLOADS["dsv3_rank"]
    Rs = [int(r) for r in args.eplb.split(",")]
    S_max = (base.E + max(Rs)) // G
    wl = base.replace(name="deepseek_v3_T16384_d7168_E256_k8_F2048_fp8_zipf1.2", num_local=S_max)
    pr = synth.make_problem(wl)
    x_meas = pr.x.to(dev)
    x_win = synth.tokens(wl, seed=1000 + wl.seed).to(dev)
    wr = pr.w_router.to(dev)
    bias = pr.bias.to(dev)
    W = {n: getattr(pr, n).to(dev) for n in ("w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down")}
    T, d, E, k, F = wl.T, wl.d, wl.E, wl.k, wl.F
    stream = torch.cuda.current_stream()

    def route(x):
        p = B.problem(T, d, E, k, F, 0, E, wl.act, wl.weight)
        logits = torch.empty((T, E), dtype=torch.float32, device=dev)
        idx = torch.empty((T, k), dtype=torch.int32, device=dev)
        gw = torch.empty((T, k), dtype=torch.float32, device=dev)
        B.moe_route(p, x, wr, bias, logits, idx, gw, ws=B.workspace(p, B.MOE_CALL_ROUTE, dev))
        counts = torch.empty((E,), dtype=torch.int32, device=dev)
        offs = torch.empty((E + 1,), dtype=torch.int32, device=dev)
        srt = torch.empty((T * k,), dtype=torch.int32, device=dev)
        pos = torch.empty((T * k,), dtype=torch.int32, device=dev)
        B.moe_permute(p, idx, counts, offs, srt, pos, B.workspace(p, B.MOE_CALL_PERMUTE, dev))
        torch.cuda.synchronize()
        return idx, gw, counts.cpu().numpy().astype(np.int64)

    _, _, window_load = route(x_win)
    idx, gw, meas_load = route(x_meas)
    print(f"[bench] eplb: routed window and measured batches; window max/mean expert load "
          f"{window_load.max() / window_load.mean():.2f}", file=sys.stderr, flush=True)
    y = torch.empty((T * k, d), dtype=pr.x.dtype, device=dev)
    out = torch.empty((T, d), dtype=pr.x.dtype, device=dev)
    steps, warmup = args.steps or 5, args.warmup if args.warmup is not None else 2

    def rank_ms(ids, P, S, g):
        p = B.problem(T, d, P, k, F, g * S, S, wl.act, wl.weight)
        counts = torch.empty((S,), dtype=torch.int32, device=dev)
        offs = torch.empty((S + 1,), dtype=torch.int32, device=dev)
        srt = torch.empty((T * k,), dtype=torch.int32, device=dev)
        pos = torch.empty((T * k,), dtype=torch.int32, device=dev)
        wsp = B.workspace(p, B.MOE_CALL_PERMUTE, dev)
        wsf = B.workspace(p, B.MOE_CALL_EXPERT_FFN, dev)

        def share():
            B.moe_permute(p, ids, counts, offs, srt, pos, wsp, stream=stream)
            B.moe_expert_ffn(p, x_meas, srt, offs, W["w_gate"], W["w_up"], W["w_down"],
                             W["s_gate"], W["s_up"], W["s_down"], gw, y, wsf, stream=stream)
            B.moe_combine(p, y, pos, None, out, stream=stream)

        for _ in range(warmup):
            share()
        ts = []
        for _ in range(steps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            share()
            b.record(stream)
            b.synchronize()
            ts.append(a.elapsed_time(b))
        return float(np.median(ts)), int(counts.sum().item())

    base_max = None
    for label, R in [("contiguous", None)] + [(f"eplb_R{r}", r) for r in Rs]:
        if R is None:
            P, S = E, E // G
            ids, rep_plan, remap_ms = idx, None, 0.0
            planned = None
        else:
            P, S = E + R, (E + R) // G
            t0 = time.perf_counter()
            rep, p2l, l2p, rl = B.moe_eplb_plan(window_load, G, R)
            plan_ms = (time.perf_counter() - t0) * 1e3
            ids = torch.empty_like(idx)
            d_rep = torch.from_numpy(rep).to(dev)
            d_l2p = torch.from_numpy(l2p).to(dev)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            B.moe_eplb_remap(T, k, E, G, idx, d_rep, d_l2p, ids, stream=stream)
            a.record(stream)
            B.moe_eplb_remap(T, k, E, G, idx, d_rep, d_l2p, ids, stream=stream)
            b.record(stream)
            b.synchronize()
            remap_ms = a.elapsed_time(b)
            rep_plan = {"max_copies": int(rep.max()), "experts_copied": int((rep > 1).sum()),
                        "plan_ms_host": round(plan_ms, 3)}
            planned = float(rl.max() / rl.mean())
        per = [rank_ms(ids, P, S, g) for g in range(G)]
        ms = [m for m, _ in per]
        slots = [c for _, c in per]
        base_max = max(ms) if base_max is None else base_max
        line = {"eplb": label, "workload": wl.name, "ranks": G, "redundant_experts": R or 0,
                "slots_per_rank": S, "rank_slots": slots,
                "imbalance_slots": round(max(slots) / (sum(slots) / G), 4),
                "imbalance_planned": None if planned is None else round(planned, 4),
                "rank_ms": [round(m, 4) for m in ms], "max_rank_ms": round(max(ms), 4),
                "mean_rank_ms": round(float(np.mean(ms)), 4),
                "imbalance_time": round(max(ms) / float(np.mean(ms)), 4),
                "tokens_per_s_slowest_rank": round(T / (max(ms) * 1e-3), 1),
                "speedup_vs_contiguous": round(base_max / max(ms), 4),
                "remap_ms": round(remap_ms, 5), "plan": rep_plan,
                "steps_per_rank": steps}
        print(json.dumps(line), flush=True)


def tile_rows(wl: synth.Workload) -> int:
    """M-tile height of the library's tile plan for this workload (the rows
    of one expert's segment that one tile covers)."""
    S, El = wl.T * wl.k, wl.num_local
    if wl.weight == "f32":
        return 32
    if wl.weight == "mxfp4":
        return 32 if S <= 64 * El else 128
    if S <= 16 * El or (S <= 64 * El and wl.weight == "fp8"):
        return 32
    if S < 64 * El:
        return 64
    if wl.weight == "fp8":
        return 128
    return 256 if S >= 512 * El else 128


def m_padding(wl: synth.Workload, counts: np.ndarray) -> dict:
    """Rows the expert GEMMs compute beyond the kept slots: every expert
    segment is cut into M tiles of tile_rows() rows, the last one partly
    empty.  (The N tiles divide F and d exactly at every workload shape here.)"""
    bm = tile_rows(wl)
    c = np.asarray(counts, dtype=np.int64)
    padded = int((-(-c // bm) * bm).sum())
    N = int(c.sum())
    return {"tile_rows": bm, "kept_rows": N, "computed_rows": padded,
            "padding_frac": round(1.0 - N / padded, 4) if padded else 0.0}


def summarize(wl: synth.Workload, m: dict, blocked: bool) -> dict:
    """Throughput, stage times and roofline fractions of one measured workload.

    Bases, stated with every figure: `ms_per_step_wall` is host wall time over
    back-to-back steps (no host synchronisation between them); `event_ms` is
    the spread of the per-step HIP-event brackets moe_forward records on its
    stream (each step bracketed on its own); kernel figures use the mean of
    that kernel's event bracket over the timed steps."""
    cnt = m["counts"]
    alg = algorithmic(wl, cnt, m["tokens_read"])
    t_wall = m["ms_per_step"] * 1e-3
    t_ev = float(np.median(m["layer_ev"])) * 1e-3
    st = m["stage_ms"]

    def kern(flop, nbytes, ms):
        t = ms * 1e-3
        return {"ms": round(ms, 5), "tflops": round(flop / t / 1e12, 2),
                "frac_mfma_bf16": round(flop / t / 1e12 / PEAK_BF16_TFLOPS, 4),
                "gbs": round(nbytes / t / 1e9, 1),
                "frac_hbm": round(nbytes / t / 1e9 / PEAK_HBM_GBS, 4),
                "alg_flop": int(flop), "alg_bytes": int(nbytes)}

    out = {
        "workload": wl.name, "T": wl.T, "d": wl.d, "E": wl.E, "k": wl.k, "F": wl.F,
        "local_experts": f"{wl.expert_begin}-{wl.expert_begin + wl.num_local - 1}",
        "act": wl.act, "weights": wl.weight, "weight_layout": "blocked" if blocked else "rows",
        "regime": wl.regime, "bias": list(wl.bias) if wl.bias else None,
        "ms_per_step_wall": round(m["ms_per_step"], 5),
        "tokens_per_s_wall": round(wl.T / t_wall, 1),
        "event_ms": {"p10": pct(m["layer_ev"], 10), "p50": pct(m["layer_ev"], 50),
                     "p90": pct(m["layer_ev"], 90)},
        "tokens_per_s_event_p50": round(wl.T / t_ev, 1),
        "kept_slots": alg["N"], "touched_experts": alg["touched"],
        "tokens_with_local_slot": alg["tokens_read"],
        "max_over_mean_load": round(float(cnt.max() / max(cnt.mean(), 1e-9)), 2),
        "m_padding": m_padding(wl, cnt),
        "stage_ms": {n: round(v, 5) for n, v in st.items()},
        "gate_up": kern(alg["gu_flop"], alg["gu_bytes"], st["gate_up"]),
        "down": kern(alg["dn_flop"], alg["dn_bytes"], st["down"]),
        "layer_wall": kern(alg["layer_flop"], alg["layer_bytes"], m["ms_per_step"]),
        "layer_event_p50": kern(alg["layer_flop"], alg["layer_bytes"], t_ev * 1e3),
        "weight_copies": m["copies"],
    }
    out["gate_up"]["bytes_with_h"] = alg["gu_bytes_with_h"]
    out["gate_up"]["kernel"] = gate_up_kernel_name(wl, blocked)
    if wl.weight == "fp8":
        out["gate_up"]["frac_mfma_fp8"] = round(alg["gu_flop"] / (st["gate_up"] * 1e-3) / 1e12
                                                / PEAK_FP8_TFLOPS, 4)
    if m["warm_ms"] is not None:
        out["warm_ms_per_step"] = round(m["warm_ms"], 5)
    if wl.num_local < wl.E:
        # one expert-parallel rank's share: routing all T tokens over all E
        # experts is setup shared by the ranks; the share is permute .. combine
        t_share = float(np.median(m["share_ev"])) * 1e-3
        out["rank_share"] = {
            "ms_p50": round(t_share * 1e3, 5), "tokens_per_s": round(wl.T / t_share, 1),
            "kept_slots_per_s": round(alg["N"] / t_share, 1),
            "tflops": round(alg["expert_flop"] / t_share / 1e12, 2),
            "gbs": round(alg["expert_bytes"] / t_share / 1e9, 1),
            "frac_mfma_bf16": round(alg["expert_flop"] / t_share / 1e12 / PEAK_BF16_TFLOPS, 4),
            "frac_hbm": round(alg["expert_bytes"] / t_share / 1e9 / PEAK_HBM_GBS, 4)}
    return out


# Workloads measured beside the headline in the default run (each timed with
# fewer steps: they are compute-bound or large, and the whole command must stay
# within a few minutes).
EXTRA_CONFIGS = ["tiny", "decode_mxfp4", "prefill", "prefill_cal", "prefill_mxfp4", "mixtral",
                 "dsv3_rank", "dsv3_rank_4k"]


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--config", default="decode", choices=sorted(synth.WORKLOADS))
    ap.add_argument("--configs", default=None,
                    help="comma-separated workloads measured beside the headline one and "
                         "reported under 'configs' ('none' for none; default: all others when "
                         "the headline is the decode step)")
    ap.add_argument("--weight-copies", type=int, default=None)
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--layout", default="blocked", choices=("rows", "blocked"),
                    help="expert weight layout: converted once (untimed, as at model load) to "
                         "the library's blocked layout (default), or row-major")
    ap.add_argument("--eplb", default=None,
                    help="comma-separated redundant-expert counts: EPLB placements of the "
                         "DeepSeek-V3 layer on 8 ranks (one JSON line per placement)")
    ap.add_argument("--sweep", default=None,
                    help="comma-separated token counts: batch sweep at the Qwen3 shape "
                         "(one JSON line per T instead of the bench line)")
    ap.add_argument("--dense-ref", action="store_true",
                    help="reference only: torch.matmul (hipBLASLt) on dense bf16 GEMMs of the "
                         "prefill workloads' expert-GEMM shapes (one JSON line per GEMM)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's share of the MoE layer: only --gpus 1 is supported "
              "(expert-parallel sharding across GPUs is not built).", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    B.load_library()
    if args.sweep:
        sweep(args, dev)
        return
    if args.eplb:
        eplb(args, dev)
        return
    if args.dense_ref:
        dense_ref(args, dev)
        return

    wl = synth.WORKLOADS[args.config]
    steps = args.steps or (200 if wl.regime in ("decode", "tiny") else 50)
    warmup = args.warmup if args.warmup is not None else 10
    # at least four weight copies rotate through the steps, so that no step
    # finds a previous step's weights in the 256 MB Infinity Cache
    copies = args.weight_copies or 4
    blocked = args.layout == "blocked" and wl.weight != "f32"
    m = measure(wl, steps, warmup, copies, dev, blocked)
    pr = m["pr"]
    sm = summarize(wl, m, blocked)
    decode = wl.regime in ("decode", "tiny")
    gu = sm["gate_up"]
    if decode:
        roof = {"bound": "hbm", "achieved": gu["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": gu["frac_hbm"], "traffic": None}
    else:
        peak = PEAK_FP32_TFLOPS if wl.weight == "f32" else PEAK_BF16_TFLOPS
        roof = {"bound": "mfma", "achieved": gu["tflops"], "peak": peak, "unit": "TFLOP/s",
                "frac": round(gu["tflops"] / peak, 4), "traffic": None}
        if wl.weight == "fp8":
            roof["frac_of_fp8_peak"] = gu["frac_mfma_fp8"]
    roof["kernel"] = gu["kernel"]
    roof["traffic"] = measured_traffic(wl.name, roof["kernel"], "blocked" if blocked else "rows")
    roof["basis"] = ("the gate/up grouped GEMM alone: algorithmic bytes (weights of the touched "
                     "experts and the token rows, without the materialised h) or FLOPs per "
                     "launch over the mean of its HIP-event bracket on the library's stream")
    roof["kernel_ms"] = gu["ms"]
    roof["bytes_per_launch"] = gu["alg_bytes"]
    roof["bytes_per_launch_with_h"] = gu["bytes_with_h"]
    roof["flop_per_launch"] = gu["alg_flop"]

    lw, le = sm["layer_wall"], sm["layer_event_p50"]
    layer = {"tflops": lw["tflops"], "gbs": lw["gbs"], "frac_hbm": lw["frac_hbm"],
             "frac_mfma_bf16": lw["frac_mfma_bf16"],
             "basis": "ms_per_step: host wall time over back-to-back steps",
             "event_p50": {"ms": le["ms"], "frac_hbm": le["frac_hbm"],
                           "frac_mfma_bf16": le["frac_mfma_bf16"],
                           "basis": "median of the per-step HIP-event brackets"},
             "kept_slots": sm["kept_slots"],
             "kept_slots_per_s": round(sm["kept_slots"] / (m["ms_per_step"] * 1e-3), 1),
             "touched_experts": sm["touched_experts"],
             "tokens_with_local_slot": sm["tokens_with_local_slot"],
             "max_over_mean_load": sm["max_over_mean_load"], "m_padding": sm["m_padding"],
             "stage_ms": sm["stage_ms"], "event_ms_per_step": sm["event_ms"],
             "warm_ms_per_step": sm.get("warm_ms_per_step")}
    if "rank_share" in sm:
        layer["rank_share"] = sm["rank_share"]

    result = {
        "metric": METRIC,
        "value": sm["tokens_per_s_wall"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": sm["ms_per_step_wall"],
        "ms_per_step_basis": "host wall time over back-to-back steps",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"fp8": "bf16 (fp8-e4m3 weights)", "mxfp4": "bf16 (mxfp4 weights)"}.get(
            wl.weight, wl.act),
        "data": "synthetic (seeded; random-init weights of the workload's shape)",
        "config": {"workload": wl.name, "T": wl.T, "d": wl.d, "E": wl.E, "k": wl.k, "F": wl.F,
                   "local_experts": sm["local_experts"], "act": wl.act, "weights": wl.weight,
                   "weight_copies": copies, "weight_layout": sm["weight_layout"],
                   "parallelism": "single GPU (all experts local)" if wl.num_local == wl.E
                   else "one expert-parallel rank's expert block"},
        "layer": layer,
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(pr, m["logits"], args.cpu_budget)
    del m, pr

    extra = (EXTRA_CONFIGS if args.config == "decode" else []) if args.configs is None else \
        [c for c in args.configs.split(",") if c and c != "none"]
    if extra:
        cfgs = {}
        for name in extra:
            if name == args.config:
                continue
            ewl = synth.WORKLOADS[name]
            dec = ewl.regime in ("decode", "tiny")
            # fixed, small step counts (a few ms of GPU time each): the
            # headline's --steps / --warmup do not apply to these lines
            esteps, ewarm = (40, 10) if dec else (20, 5)
            eblocked = args.layout == "blocked" and ewl.weight != "f32"
            print(f"[bench] config {name}: generating", file=sys.stderr, flush=True)
            em = measure(ewl, esteps, ewarm, 4 if dec else 2, dev, eblocked, warm=False)
            es = summarize(ewl, em, eblocked)
            es["steps"], es["warmup"] = esteps, ewarm
            es["gate_up"]["traffic"] = measured_traffic(ewl.name, es["gate_up"]["kernel"],
                                                        es["weight_layout"])
            if not args.no_cpu_baseline:
                es["cpu_baseline"] = cpu_baseline(em["pr"], em["logits"], 2.0, n_sample=16)
            cfgs[name] = es
            del em
            torch.cuda.empty_cache()
            print(f"[bench] config {name}: {es['ms_per_step_wall']} ms/step, gate/up "
                  f"{es['gate_up']['frac_mfma_bf16']:.3f} MFMA / {es['gate_up']['frac_hbm']:.3f} "
                  "HBM", file=sys.stderr, flush=True)
        result["configs"] = cfgs
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
