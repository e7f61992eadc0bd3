"""Thin ctypes binding of the C ABI in ``include/moe.h``.

Argument marshalling only: tensors become device pointers, the stream becomes
the current HIP stream, status codes become exceptions.  Every step of the
layer runs in the HIP library; there is no fallback of any kind.  PyTorch is
used for device memory and streams.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("MOE_MI355X_LIB", os.path.join(PKG, "libmoe_mi355x.so"))

MOE_OK, MOE_ERR_INVALID_ARGUMENT, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE_TOO_SMALL, MOE_ERR_HIP = range(5)
MOE_F32, MOE_BF16, MOE_FP8_E4M3, MOE_MXFP4 = range(4)
MOE_CALL_PERMUTE, MOE_CALL_EXPERT_FFN, MOE_CALL_FORWARD, MOE_CALL_ROUTE = range(4)
MOE_FORWARD_EVENTS = 7
MOE_LAYOUT_ROWS, MOE_LAYOUT_BLOCKED = range(2)
MOE_NOALLOC_SCRATCH_BYTES = 64 << 20   # include/moe.h

FMT = {"f32": MOE_F32, "bf16": MOE_BF16, "fp8": MOE_FP8_E4M3, "mxfp4": MOE_MXFP4}


class MoEError(RuntimeError):
    def __init__(self, call: str, status: int, text: str):
        super().__init__(f"{call} failed: {text} ({status})")
        self.status = status


class Problem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("T", "d", "E", "k", "F", "expert_begin", "num_local", "act", "weight",
                 "weight_layout")]


class ForwardArgs(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("x", "w_router", "router_bias", "w_gate", "w_up", "w_down", "s_gate", "s_up",
                 "s_down", "out", "logits", "topk_idx", "topk_w", "counts", "offsets",
                 "sorted_slot", "slot_pos", "events")]


_lib = None


def load_library() -> ctypes.CDLL:
    """Load the built library; raise if it is missing (no fallback exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it first with "
                          "`python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
    P = ctypes.POINTER(Problem)
    lib.moe_workspace_size.argtypes = [P, i32]
    lib.moe_workspace_size.restype = sz
    lib.moe_status_string.argtypes = [ctypes.c_int]
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_route.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.moe_permute.argtypes = [P, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.moe_expert_ffn.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.moe_combine.argtypes = [P, vp, vp, vp, vp, vp]
    lib.moe_forward.argtypes = [P, ctypes.POINTER(ForwardArgs), vp, sz, vp]
    lib.moe_forward_noalloc.argtypes = [P, ctypes.POINTER(ForwardArgs), vp]
    i64p, i32p, f64p = (ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int32),
                        ctypes.POINTER(ctypes.c_double))
    lib.moe_eplb_plan.argtypes = [i64p, i32, i32, i32, i32p, i32p, i32p, f64p]
    lib.moe_eplb_remap.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, vp]
    lib.moe_pack_weights.argtypes = [P, i32, vp, vp, vp]
    for f in ("moe_route", "moe_permute", "moe_expert_ffn", "moe_combine", "moe_forward",
              "moe_forward_noalloc", "moe_eplb_plan", "moe_eplb_remap", "moe_pack_weights"):
        getattr(lib, f).restype = ctypes.c_int
    _lib = lib
    return lib


def problem(T, d, E, k, F, expert_begin=0, num_local=None, act="bf16", weight="bf16",
            blocked=False) -> Problem:
    num_local = E - expert_begin if num_local is None else num_local
    return Problem(T, d, E, k, F, expert_begin, num_local,
                   FMT[act] if isinstance(act, str) else act,
                   FMT[weight] if isinstance(weight, str) else weight,
                   MOE_LAYOUT_BLOCKED if blocked else MOE_LAYOUT_ROWS)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(call: str, status: int) -> None:
    if status != MOE_OK:
        text = load_library().moe_status_string(status).decode()
        raise MoEError(call, status, text)


def moe_status_string(status: int) -> str:
    return load_library().moe_status_string(status).decode()


def moe_workspace_size(p: Problem, call: int) -> int:
    return int(load_library().moe_workspace_size(ctypes.byref(p), call))


def moe_route(p, x, w_router, router_bias, logits, topk_idx, topk_w, ws=None,
              stream=None) -> None:
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    st = load_library().moe_route(ctypes.byref(p), _ptr(x), _ptr(w_router), _ptr(router_bias),
                                  _ptr(logits), _ptr(topk_idx), _ptr(topk_w), _ptr(ws), nbytes,
                                  _stream(stream))
    _check("moe_route", st)


def moe_permute(p, topk_idx, counts, offsets, sorted_slot, slot_pos, ws, stream=None) -> None:
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    st = load_library().moe_permute(ctypes.byref(p), _ptr(topk_idx), _ptr(counts), _ptr(offsets),
                                    _ptr(sorted_slot), _ptr(slot_pos), _ptr(ws), nbytes,
                                    _stream(stream))
    _check("moe_permute", st)


def moe_expert_ffn(p, x, sorted_slot, offsets, w_gate, w_up, w_down, s_gate, s_up, s_down,
                   topk_w, y, ws, stream=None) -> None:
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    st = load_library().moe_expert_ffn(
        ctypes.byref(p), _ptr(x), _ptr(sorted_slot), _ptr(offsets), _ptr(w_gate), _ptr(w_up),
        _ptr(w_down), _ptr(s_gate), _ptr(s_up), _ptr(s_down), _ptr(topk_w), _ptr(y), _ptr(ws),
        nbytes, _stream(stream))
    _check("moe_expert_ffn", st)


def moe_combine(p, y, slot_pos, topk_w, out, stream=None) -> None:
    st = load_library().moe_combine(ctypes.byref(p), _ptr(y), _ptr(slot_pos), _ptr(topk_w),
                                    _ptr(out), _stream(stream))
    _check("moe_combine", st)


def moe_forward(p, *, x, w_router, router_bias, w_gate, w_up, w_down, out, ws,
                s_gate=None, s_up=None, s_down=None, logits=None, topk_idx=None, topk_w=None,
                counts=None, offsets=None, sorted_slot=None, slot_pos=None, events=None,
                stream=None) -> None:
    """``events``: None, or a ctypes array of MOE_FORWARD_EVENTS hipEvent_t handles."""
    a = _forward_args(x, w_router, router_bias, w_gate, w_up, w_down, out, s_gate, s_up, s_down,
                      logits, topk_idx, topk_w, counts, offsets, sorted_slot, slot_pos, events)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    st = load_library().moe_forward(ctypes.byref(p), ctypes.byref(a), _ptr(ws), nbytes,
                                    _stream(stream))
    _check("moe_forward", st)


def _forward_args(x, w_router, router_bias, w_gate, w_up, w_down, out, s_gate, s_up, s_down,
                  logits, topk_idx, topk_w, counts, offsets, sorted_slot, slot_pos, events):
    return ForwardArgs(_ptr(x), _ptr(w_router), _ptr(router_bias), _ptr(w_gate), _ptr(w_up),
                       _ptr(w_down), _ptr(s_gate), _ptr(s_up), _ptr(s_down), _ptr(out),
                       _ptr(logits), _ptr(topk_idx), _ptr(topk_w), _ptr(counts), _ptr(offsets),
                       _ptr(sorted_slot), _ptr(slot_pos),
                       None if events is None else ctypes.addressof(events))


def moe_forward_noalloc(p, *, x, w_router, router_bias, w_gate, w_up, w_down, out,
                        s_gate=None, s_up=None, s_down=None, logits=None, topk_idx=None,
                        topk_w=None, counts=None, offsets=None, sorted_slot=None, slot_pos=None,
                        events=None, stream=None) -> None:
    """moe_forward with the library's own scratch array (no workspace argument)."""
    a = _forward_args(x, w_router, router_bias, w_gate, w_up, w_down, out, s_gate, s_up, s_down,
                      logits, topk_idx, topk_w, counts, offsets, sorted_slot, slot_pos, events)
    st = load_library().moe_forward_noalloc(ctypes.byref(p), ctypes.byref(a), _stream(stream))
    _check("moe_forward_noalloc", st)


def moe_eplb_plan(load, G: int, R: int):
    """Host placement plan (see moe.h).  ``load``: per-expert counts (any
    integer sequence).  Returns numpy ``(replicas [E], phys_to_log [E+R],
    log_to_phys [E, G], rank_load [G])``."""
    import numpy as np
    ld = np.ascontiguousarray(np.asarray(load, dtype=np.int64))
    E = int(ld.shape[0])
    rep = np.zeros(E, dtype=np.int32)
    p2l = np.zeros(max(E + R, 1), dtype=np.int32)
    l2p = np.zeros((E, max(G, 1)), dtype=np.int32)
    rl = np.zeros(max(G, 1), dtype=np.float64)
    c = ctypes
    st = load_library().moe_eplb_plan(
        ld.ctypes.data_as(c.POINTER(c.c_int64)), E, G, R,
        rep.ctypes.data_as(c.POINTER(c.c_int32)), p2l.ctypes.data_as(c.POINTER(c.c_int32)),
        l2p.ctypes.data_as(c.POINTER(c.c_int32)), rl.ctypes.data_as(c.POINTER(c.c_double)))
    _check("moe_eplb_plan", st)
    return rep, p2l, l2p, rl


def moe_eplb_remap(T, k, E, G, topk_idx, replicas, log_to_phys, topk_phys, stream=None) -> None:
    st = load_library().moe_eplb_remap(T, k, E, G, _ptr(topk_idx), _ptr(replicas),
                                       _ptr(log_to_phys), _ptr(topk_phys), _stream(stream))
    _check("moe_eplb_remap", st)


def moe_pack_weights(p, which: int, src, dst, stream=None) -> None:
    """Blocked layout of one expert matrix set (which 0: gate or up, 1: down)."""
    st = load_library().moe_pack_weights(ctypes.byref(p), which, _ptr(src), _ptr(dst),
                                         _stream(stream))
    _check("moe_pack_weights", st)


def workspace(p: Problem, call: int, device="cuda") -> torch.Tensor:
    """A device scratch tensor of the size the library asks for (torch memory)."""
    n = moe_workspace_size(p, call)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)
