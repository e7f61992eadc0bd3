"""Plain float64 CPU oracle of one mixture-of-experts (MoE) layer's forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (no kernels, headers, helpers or tables); both sides receive the same
seeded inputs and nothing else.

What the layer computes, and where the pages say so
---------------------------------------------------
* "Wide Expert Parallelism" (kodekloud llm-d notes), section "What is an MoE
  layer?": a layer holds many independent expert sub-networks and a small
  routing gate; the gate looks at each token and sends it to a small subset
  of the experts (DeepSeek-R1: 8 of 256), the others stay idle for it.
* "Expert Parallelism for MoE Models" (apxml), section "Mechanics of Token
  Routing and All-to-All Communication": a routing layer assigns each token
  to one or more experts; the token's representation is sent to where the
  expert lives, the expert computes, and the result is sent back.
* "Serving MoE models with expert parallelism on 8xH200" (reviosa), section
  "Tensor parallel vs expert parallel": each GPU owns whole experts (256
  routed experts on 8 GPUs gives 32 each) and runs full-size expert GEMMs on
  the tokens dispatched to it.

The pages leave the gate's exact form, the expert network and the combine
open.  The readings taken here (all exact, no approximation):
* router logits ``L = x . W_r + b`` (``b`` a per-expert logit bias, zero when
  absent);
* top-k by the key ``(-L[t,e], e)``: the k largest logits, ties to the lower
  expert index, listed in that order;
* gates = softmax over all E experts, then renormalised over the k chosen;
  the full-E denominator cancels, so ``w_i = exp(L_i - m) / sum_j exp(L_j - m)``
  over the chosen j, with ``m`` the largest chosen logit;
* each expert is a SwiGLU feed-forward network without biases,
  ``FFN_e(x) = (silu(x . Wg_e) * (x . Wu_e)) . Wd_e``, ``silu(z) = z * sigmoid(z)``
  (Shazeer 2020, "GLU Variants Improve Transformer");
* combine: ``out[t] = sum_i w[t,i] * FFN_{idx[t,i]}(x[t])`` in i order; on an
  expert-parallel rank only the slots whose expert lies in the rank's block
  ``[e0, e0+E_l)`` contribute, and a token with none of them gets 0;
* dispatch is a stable counting sort of the kept slots ``s = t*k + i`` by
  expert: per-expert counts, their exclusive prefix sum, and the slots of each
  expert in increasing slot order.

Storage conventions of the inputs (shared with the library's C ABI):
* activations ``x [T, d]``: ``"f32"`` float32, or ``"bf16"`` as uint16 bit
  patterns;
* router ``w_router [d, E]`` in the activation format, ``bias [E]`` float32;
* expert weights stored "out x in": ``w_gate, w_up [E_l, F, d]`` and
  ``w_down [E_l, d, F]``, i.e. the math matrices ``Wg_j, Wu_j [d, F]`` and
  ``Wd_j [F, d]`` transposed; ``"f32"``, ``"bf16"`` (uint16 bits) or ``"fp8"``
  (uint8 OCP E4M3FN codes) with float32 scales per 128x128 block of the
  stored matrix: ``s_gate, s_up [E_l, F/128, d/128]``, ``s_down [E_l, d/128, F/128]``.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_bits_to_f64", "e4m3fn_table", "e4m3fn_to_f64", "dequant_block128",
    "e2m1_table", "e8m0_to_f64", "dequant_mxfp4",
    "decode_act", "decode_expert_weight", "router_logits", "topk_select",
    "renormalised_gates", "local_slot_mask", "expert_permutation",
    "silu", "swiglu_ffn", "moe_layer_forward", "routed_layer_forward", "brute_force_dense",
]

BLOCK = 128  # side of the square fp8 scale block


# ----------------------------------------------------------------------------
# Exact decoding of the stored number formats
# ----------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float64, exactly.

    bfloat16 is the upper half of an IEEE-754 binary32, so placing the 16 bits
    above 16 zero bits gives the binary32 value, which float64 holds exactly.
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):      # NaN patterns stay NaN
        return b.view(np.float32).astype(np.float64)


def e4m3fn_table() -> np.ndarray:
    """All 256 OCP FP8 E4M3FN codes -> float64.

    The format (OCP 8-bit floating point specification, E4M3 variant):
    1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0
    encodes subnormals ``(m/8) * 2^-6``; there is no infinity, and only
    ``S.1111.111`` is NaN, so the largest finite magnitude is ``1.75 * 2^8 = 448``.
    """
    out = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            out[code] = np.nan
        elif e == 0:
            out[code] = sign * (m / 8.0) * 2.0 ** (1 - 7)
        else:
            out[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return out


_E4M3 = e4m3fn_table()


def e4m3fn_to_f64(codes: np.ndarray) -> np.ndarray:
    """OCP E4M3FN codes (uint8) -> float64 via the 256-entry table."""
    return _E4M3[np.asarray(codes, dtype=np.uint8)]


def dequant_block128(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """``W[r, c] = e4m3(q[r, c]) * s[r // 128, c // 128]`` for one stored matrix.

    "Serving MoE models with expert parallelism on 8xH200", section
    "Quantization choices", names native FP8 expert weights; the 128x128 block
    granularity of the float32 scales is the reading used for the
    DeepSeek-V3-shaped workload.
    """
    q = np.asarray(q)
    R, C = q.shape
    assert R % BLOCK == 0 and C % BLOCK == 0
    assert s.shape == (R // BLOCK, C // BLOCK)
    w = e4m3fn_to_f64(q).reshape(R // BLOCK, BLOCK, C // BLOCK, BLOCK)
    w *= np.asarray(s, dtype=np.float64)[:, None, :, None]   # s[r // 128, c // 128]
    return w.reshape(R, C)


MX_BLOCK = 32  # elements sharing one E8M0 scale in an MXFP4 row


def e2m1_table() -> np.ndarray:
    """All 16 OCP FP4 E2M1 codes -> float64.

    The format (OCP Microscaling Formats (MX) specification v1.0, FP4 E2M1
    element): 1 sign bit (bit 3), 2 exponent bits (bits 2..1) with bias 1, 1
    mantissa bit (bit 0); exponent field 0 encodes the subnormal ``m * 0.5``;
    no infinity or NaN, so magnitudes run 0, 0.5, 1, 1.5, 2, 3, 4, 6.
    """
    out = np.empty(16, dtype=np.float64)
    for code in range(16):
        sign = -1.0 if code & 0x8 else 1.0
        e = (code >> 1) & 0x3
        m = code & 0x1
        out[code] = sign * (m * 0.5 if e == 0 else (1.0 + m / 2.0) * 2.0 ** (e - 1))
    return out


_E2M1 = e2m1_table()


def e8m0_to_f64(s: np.ndarray) -> np.ndarray:
    """OCP E8M0 scale bytes -> float64: ``2^(s - 127)``; 255 is NaN."""
    s = np.asarray(s, dtype=np.int64)
    return np.where(s == 255, np.nan, np.ldexp(1.0, s - 127))


def dequant_mxfp4(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """One MXFP4 matrix -> float64 ``[R, C]``.

    ``q [R, C/2]`` uint8: byte j of a row holds element 2j in bits 0..3 and
    element 2j+1 in bits 4..7; ``s [C/32, R]`` uint8 E8M0 scales, stored
    block-major (all rows' scales of K block b are contiguous);
    ``W[r, c] = e2m1(element c of row r) * 2^(s[c // 32, r] - 127)``.
    "Serving MoE models with expert parallelism on 8xH200": section "Memory
    math for 8xH200" names gpt-oss-120b in its native MXFP4, section
    "Quantization choices" 4-bit expert weights that halve the footprint of
    FP8 again.
    """
    q = np.asarray(q, dtype=np.uint8)
    R, half = q.shape
    C = 2 * half
    assert C % MX_BLOCK == 0 and s.shape == (C // MX_BLOCK, R)
    codes = np.empty((R, C), dtype=np.uint8)
    codes[:, 0::2] = q & 0x0F
    codes[:, 1::2] = q >> 4
    w = _E2M1[codes].reshape(R, C // MX_BLOCK, MX_BLOCK)
    w *= e8m0_to_f64(s).T[:, :, None]   # s[c // 32, r]
    return w.reshape(R, C)


def decode_act(a: np.ndarray, fmt: str) -> np.ndarray:
    """Activation / router storage -> float64 (``"f32"`` or ``"bf16"`` bits)."""
    if fmt == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if fmt == "bf16":
        return bf16_bits_to_f64(a)
    raise ValueError(f"unknown activation format {fmt!r}")


def decode_expert_weight(w: np.ndarray, fmt: str, scale: np.ndarray | None = None) -> np.ndarray:
    """One stored expert matrix ("out x in") -> float64 in the same orientation."""
    if fmt == "f32":
        return np.asarray(w, dtype=np.float32).astype(np.float64)
    if fmt == "bf16":
        return bf16_bits_to_f64(w)
    if fmt == "fp8":
        return dequant_block128(w, scale)
    if fmt == "mxfp4":
        return dequant_mxfp4(w, scale)
    raise ValueError(f"unknown weight format {fmt!r}")


# ----------------------------------------------------------------------------
# Routing ("What is an MoE layer?": the gate picks a small subset per token)
# ----------------------------------------------------------------------------

def router_logits(x64: np.ndarray, w_router64: np.ndarray, bias: np.ndarray | None) -> np.ndarray:
    """``L = x . W_r + b`` in float64; ``x [T,d]``, ``W_r [d,E]``, ``b [E]``."""
    L = x64 @ w_router64
    if bias is not None:
        L = L + np.asarray(bias, dtype=np.float64)[None, :]
    return L


def topk_select(L: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest logits per row, ordered by ``(-L, e)``.

    Ties between equal logits go to the lower expert index.  Comparisons are
    exact on the values given (the caller passes the float32 logits it wants
    the decision taken on).  The pages say nothing of non-finite logits; the
    reading taken (and stated in the library's contract) is that a NaN ranks
    as -inf, so it ties with -inf and with other NaNs and those ties also go to
    the lower index.  Returns int32 ``[T, k]`` of global expert ids.
    """
    L = np.asarray(L)
    T, E = L.shape
    if not 1 <= k <= E:
        raise ValueError("k must lie in [1, E]")
    L = np.where(np.isnan(L), -np.inf, L)
    experts = np.broadcast_to(np.arange(E), L.shape)
    order = np.lexsort((experts, -L), axis=-1)  # last key is primary
    return order[:, :k].astype(np.int32)


def renormalised_gates(L: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Softmax over the experts, renormalised over each token's k chosen.

    With ``p_e = exp(L_e) / sum_all exp(L)``, the renormalised gate is
    ``p_i / sum_{j chosen} p_j``; the full sum cancels, leaving a softmax over
    the chosen logits.  ``m`` (the first, largest chosen logit) is subtracted
    for range only.  float64 ``[T, k]``.
    """
    Lc = np.take_along_axis(np.asarray(L, dtype=np.float64), idx.astype(np.int64), axis=1)
    m = Lc[:, :1]
    e = np.exp(Lc - m)
    return e / e.sum(axis=1, keepdims=True)


def local_slot_mask(idx: np.ndarray, e0: int, E_l: int) -> np.ndarray:
    """Flat ``[T*k]`` mask of slots ``s = t*k + i`` whose expert is in ``[e0, e0+E_l)``.

    "Tensor parallel vs expert parallel" (reviosa): with expert parallelism a
    GPU owns a block of whole experts and only computes the slots sent to them.
    """
    flat = np.asarray(idx, dtype=np.int64).reshape(-1)
    return (flat >= e0) & (flat < e0 + E_l)


def expert_permutation(idx: np.ndarray, e0: int, E_l: int):
    """Stable counting sort of the kept slots by local expert.

    Steps, in order: a histogram of kept slots per local expert; its exclusive
    prefix sum; then a pass over the slots in increasing ``s`` that drops each
    kept slot into the next free position of its expert's segment.  Returns
    ``counts [E_l]``, ``offsets [E_l+1]`` (``offsets[E_l]`` = kept count N),
    ``sorted_slot [N]`` and ``slot_pos [T*k]`` (position of each slot, -1 when
    the slot is not kept), all int32.
    """
    flat = np.asarray(idx, dtype=np.int64).reshape(-1)
    S = flat.shape[0]
    keep = local_slot_mask(idx, e0, E_l)
    counts = np.zeros(E_l, dtype=np.int64)
    for s in range(S):
        if keep[s]:
            counts[flat[s] - e0] += 1
    offsets = np.zeros(E_l + 1, dtype=np.int64)
    for j in range(E_l):
        offsets[j + 1] = offsets[j] + counts[j]
    N = int(offsets[E_l])
    cursor = offsets[:E_l].copy()
    sorted_slot = np.empty(N, dtype=np.int64)
    slot_pos = np.full(S, -1, dtype=np.int64)
    for s in range(S):
        if keep[s]:
            j = flat[s] - e0
            p = cursor[j]
            cursor[j] += 1
            sorted_slot[p] = s
            slot_pos[s] = p
    return (counts.astype(np.int32), offsets.astype(np.int32),
            sorted_slot.astype(np.int32), slot_pos.astype(np.int32))


# ----------------------------------------------------------------------------
# Experts and combine
# ----------------------------------------------------------------------------

def silu(z: np.ndarray) -> np.ndarray:
    """``silu(z) = z * sigmoid(z)``, ``sigmoid(z) = 1 / (1 + exp(-z))`` (Elfwing et al. 2018)."""
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu_ffn(X: np.ndarray, Wg: np.ndarray, Wu: np.ndarray, Wd: np.ndarray) -> np.ndarray:
    """One expert in math orientation: ``(silu(X . Wg) * (X . Wu)) . Wd``.

    ``X [n, d]``, ``Wg, Wu [d, F]``, ``Wd [F, d]``; float64 throughout.
    """
    G = X @ Wg
    U = X @ Wu
    return (silu(G) * U) @ Wd


def _expert_math(w_gate, w_up, w_down, j, weight_fmt, s_gate, s_up, s_down):
    """Decode expert j and transpose the stored "out x in" matrices to math orientation."""
    sg = None if s_gate is None else s_gate[j]
    su = None if s_up is None else s_up[j]
    sd = None if s_down is None else s_down[j]
    Wg = decode_expert_weight(w_gate[j], weight_fmt, sg).T  # [d, F]
    Wu = decode_expert_weight(w_up[j], weight_fmt, su).T    # [d, F]
    Wd = decode_expert_weight(w_down[j], weight_fmt, sd).T  # [F, d]
    return Wg, Wu, Wd


def moe_layer_forward(x, logits, k, w_gate, w_up, w_down, *, act_fmt, weight_fmt,
                      e0=0, E_l=None, s_gate=None, s_up=None, s_down=None, tokens=None):
    """The whole layer on one GPU's share, routed from the given logits.

    ``logits [T, E]`` are the values the top-k decision is taken on (the
    library's float32 logits when checking it, so that both sides decide on
    identical numbers).  Experts are evaluated one at a time over the set of
    tokens that chose them; no grouped buffer is built.  ``tokens`` restricts
    the output rows computed (routing and permutation are always complete).

    Returns a dict with ``topk_idx``, ``topk_w`` (float64), ``counts``,
    ``offsets``, ``sorted_slot``, ``slot_pos`` and ``out`` (float64 rows for
    ``tokens``, or all T rows), plus ``tokens``.
    """
    L = np.asarray(logits)
    T, E = L.shape
    if E_l is None:
        E_l = E - e0
    idx = topk_select(L, k)
    w = renormalised_gates(L, idx)
    return routed_layer_forward(x, idx, w, w_gate, w_up, w_down, act_fmt=act_fmt,
                                weight_fmt=weight_fmt, e0=e0, E_l=E_l, s_gate=s_gate, s_up=s_up,
                                s_down=s_down, tokens=tokens)


def routed_layer_forward(x, idx, w, w_gate, w_up, w_down, *, act_fmt, weight_fmt, e0, E_l,
                         s_gate=None, s_up=None, s_down=None, tokens=None):
    """The layer's dispatch, experts and combine for given routing: expert ids
    ``idx [T, k]`` (ids outside the block ``[e0, e0+E_l)`` are not local) and
    gates ``w [T, k]``.  Same outputs as ``moe_layer_forward``."""
    x64_all = None
    T, k = idx.shape
    counts, offsets, sorted_slot, slot_pos = expert_permutation(idx, e0, E_l)

    tok = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    row_of = {int(t): r for r, t in enumerate(tok)}
    d = x.shape[1]
    out = np.zeros((tok.shape[0], d), dtype=np.float64)
    # per-slot expert outputs, then an ordered combine over i
    y_slot = {}
    for j in range(E_l):
        e = e0 + j
        # tokens (among those requested) that chose expert e, and at which i
        hit_t, hit_i = np.nonzero(idx[tok] == e)
        if hit_t.size == 0:
            continue
        rows = tok[hit_t]
        if x64_all is None:
            x64_all = decode_act(x, act_fmt)
        Wg, Wu, Wd = _expert_math(w_gate, w_up, w_down, j, weight_fmt, s_gate, s_up, s_down)
        Y = swiglu_ffn(x64_all[rows], Wg, Wu, Wd)
        for r, t, i in zip(range(rows.shape[0]), rows, hit_i):
            y_slot[(int(t), int(i))] = Y[r]
    for t in tok:
        acc = np.zeros(d, dtype=np.float64)
        for i in range(k):
            key = (int(t), i)
            if key in y_slot:
                acc = acc + w[t, i] * y_slot[key]
        out[row_of[int(t)]] = acc
    return dict(topk_idx=idx, topk_w=w, counts=counts, offsets=offsets,
                sorted_slot=sorted_slot, slot_pos=slot_pos, out=out, tokens=tok)


def brute_force_dense(x, logits, k, w_gate, w_up, w_down, *, act_fmt, weight_fmt,
                      e0=0, E_l=None, s_gate=None, s_up=None, s_down=None):
    """Dense masked evaluation for tiny shapes, with plain Python loops.

    Every local expert runs on every token; the result is weighted by the
    renormalised gate when the expert is among the token's k chosen and by 0
    otherwise.  The chosen set comes from a selection loop (repeatedly take
    the largest remaining logit, lower index first on ties), not a sort.
    Returns float64 ``[T, d]``.
    """
    L = np.asarray(logits, dtype=np.float64)
    T, E = L.shape
    if E_l is None:
        E_l = E - e0
    x64 = decode_act(x, act_fmt)
    d = x64.shape[1]
    out = np.zeros((T, d), dtype=np.float64)
    experts = [_expert_math(w_gate, w_up, w_down, j, weight_fmt, s_gate, s_up, s_down)
               for j in range(E_l)]
    for t in range(T):
        chosen = []
        for _ in range(k):
            best = None
            for e in range(E):
                if e in chosen:
                    continue
                if best is None or L[t, e] > L[t, best]:
                    best = e
            chosen.append(best)
        z = [np.exp(L[t, e] - L[t, chosen[0]]) for e in chosen]
        tot = sum(z)
        gate = [0.0] * E
        for e, ze in zip(chosen, z):
            gate[e] = ze / tot
        for j in range(E_l):
            Wg, Wu, Wd = experts[j]
            xt = x64[t:t + 1]
            out[t] += gate[e0 + j] * swiglu_ffn(xt, Wg, Wu, Wd)[0]
    return out
