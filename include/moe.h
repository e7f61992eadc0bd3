/*
 * moe.h - C ABI of the MI355X (gfx950) mixture-of-experts layer forward.
 *
 * One MoE layer on one GPU's share of the work: router logits, softmax top-k
 * gating, dispatch of token slots into expert-sorted order, each local
 * expert's SwiGLU feed-forward network as a grouped GEMM over ragged
 * per-expert segments, and the gate-weighted combine back to token order.
 * The share is either all E experts, or one expert-parallel rank's block of
 * E_l consecutive experts [expert_begin, expert_begin + E_l) seeing all T
 * tokens.
 *
 * Where the operations come from:
 *  - "Wide Expert Parallelism" (llm-d notes, kodekloud), section "What is an
 *    MoE layer?": a small gate looks at each token and routes it to a small
 *    subset of many independent experts (DeepSeek-R1: 8 of 256).
 *  - "Expert Parallelism for MoE Models" (apxml), section "Mechanics of Token
 *    Routing and All-to-All Communication": the token representation travels
 *    to where its expert lives, the expert computes, the output travels back.
 *  - "Serving MoE models with expert parallelism on 8xH200" (reviosa),
 *    section "Tensor parallel vs expert parallel": a GPU owns whole experts
 *    (256 on 8 GPUs: 32 each) and runs full-size expert GEMMs on the tokens
 *    dispatched to it.
 * The pages fix neither the gate formula nor the expert network.  This
 * library computes (exactly, up to floating-point rounding):
 *    L[t,e]   = sum_c x[t,c] W_r[c,e] + b[e]                 (float32 accumulate)
 *    idx[t,:] = the k experts with the largest L[t,.], ordered by (-L, e):
 *               ties go to the lower expert index
 *    w[t,i]   = exp(L[t,idx_i] - m) / sum_j exp(L[t,idx_j] - m), m = L[t,idx_0]
 *               (softmax over all E, renormalised over the k chosen)
 *    FFN_e(v) = (silu(v Wg_e) * (v Wu_e)) Wd_e,   silu(z) = z / (1 + exp(-z))
 *    out[t]   = sum_{i < k, idx[t,i] local} w[t,i] FFN_{idx[t,i]}(x[t])   (in i order)
 *
 * Conventions for every call
 *  - All device arrays are row-major, 16-byte aligned, owned by the caller
 *    and must stay valid until the stream work completes.  The library never
 *    allocates, frees or synchronises, and keeps no state between calls:
 *    every call queries the device it launches on, and the only thing it
 *    remembers is, per kernel and device, that the kernel's LDS-size
 *    attribute has been set (an idempotent setting recorded in an atomic bit
 *    set).  Calls are therefore re-entrant and may run concurrently from
 *    several host threads (on distinct workspaces and outputs).  Scratch
 *    memory comes from the caller (moe_workspace_size).
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Every call only enqueues kernels on it and returns.
 *  - The environment variable MOE_MI355X_MAX_WORKGROUPS, if set to a positive
 *    number, caps the workgroups of the persistent expert GEMM kernels (a
 *    test aid; results are the same for every value).  Results are
 *    deterministic: the same inputs on the same device give the same bits.
 *    The prefill-sized expert GEMMs cut the items of their last partial wave
 *    along K by the device's compute-unit count, so their float32 sums (not
 *    the routing or dispatch) may round differently on a device with another
 *    count.
 *  - A slot is s = t*k + i (token t, its i-th chosen expert).  Expert ids in
 *    index arrays are global ids in [0, E).
 *  - Formats: activations and the router matrix are MOE_F32 or MOE_BF16;
 *    expert weights are MOE_F32, MOE_BF16, MOE_FP8_E4M3 (OCP E4M3FN codes,
 *    one byte each) with float32 scales per 128x128 block of the stored
 *    matrix, or MOE_MXFP4 (OCP MX FP4: E2M1 codes, two per byte along the
 *    "in" dimension, element 2j in the low nibble of byte j, with one E8M0
 *    scale byte 2^(s-127) per 32 consecutive "in" values).  Supported
 *    (act, weight) pairs: (F32, F32), (BF16, BF16), (BF16, FP8_E4M3),
 *    (BF16, MXFP4).  Accumulation is float32; intermediate h is rounded to
 *    the activation format.  FP8 block scales are finite, and each is 0 (the
 *    block contributes nothing) or between 2^-100 and 2^100 in magnitude.
 *    The GEMMs fold them in by rescaling a float32 accumulator from one
 *    128-deep K block to the next (it holds the running sum divided by the
 *    latest nonzero scale), which bounds the inputs: the nonzero scales that
 *    one output feature meets along K (one row of the [F/128][d/128] or
 *    [d/128][F/128] scale grid) lie within a factor of 2^32 of each other,
 *    and x and the intermediate h are at most 2^64 in magnitude, so that no
 *    rescaled partial sum can leave the float32 range; outputs beyond the
 *    bfloat16 range are outside the contract.  MXFP4 weights are widened exactly to
 *    bfloat16 with their scale applied, which holds for scale bytes 0..252
 *    (2^-127 .. 2^125); bytes 253..255 are outside the contract.
 *  - Expert weights are stored "out x in" (the math matrices transposed):
 *      w_gate, w_up : [E_l][F][d]      w_down : [E_l][d][F]
 *    (MXFP4: [E_l][F][d/2] and [E_l][d][F/2] bytes), with scales
 *      FP8:   s_gate, s_up : [E_l][F/128][d/128]   s_down : [E_l][d/128][F/128]  float32
 *      MXFP4: s_gate, s_up : [E_l][d/32][F]        s_down : [E_l][F/32][d]       uint8 E8M0
 *    (MXFP4 scales are stored K-block-major: the scales of one 32-value block
 *    of all rows are contiguous), so that Wg_e[c][f] =
 *    w_gate[e - expert_begin][f][c] times its scale.
 *
 * Errors: every call checks its arguments on the host before enqueuing
 * anything and returns MOE_ERR_INVALID_ARGUMENT (null required pointer, a
 * size out of range, d or F not a multiple of 128, expert_begin + num_local
 * > E), MOE_ERR_UNSUPPORTED (an unsupported format pair or a size above the
 * stated limits) or MOE_ERR_WORKSPACE_TOO_SMALL.  A failed kernel launch
 * returns MOE_ERR_HIP.  On a device, an expert id outside [0, E) in a
 * caller-supplied topk_idx is treated as not local (it never faults).  No
 * C++ exception crosses this interface.
 *
 * Limits: 1 <= k <= E <= 512; T*k < 2^31; d, F multiples of 128 and
 * at most 65536; x (T*d elements) and one expert's weight matrix (F*d
 * elements) under 4 GiB each; T = 0 is accepted and enqueues nothing (no
 * output is written).
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = 1,
  MOE_ERR_UNSUPPORTED = 2,
  MOE_ERR_WORKSPACE_TOO_SMALL = 3,
  MOE_ERR_HIP = 4
} moe_status_t;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8_E4M3 = 2, MOE_MXFP4 = 3 } moe_dtype_t;

/* Which call a workspace is sized for. */
typedef enum {
  MOE_CALL_PERMUTE = 0,
  MOE_CALL_EXPERT_FFN = 1,
  MOE_CALL_FORWARD = 2,
  MOE_CALL_ROUTE = 3
} moe_call_t;

/* Layout of the expert weight matrices. */
typedef enum {
  MOE_LAYOUT_ROWS = 0,    /* "out x in" row-major, as described above */
  MOE_LAYOUT_BLOCKED = 1  /* the blocked layout written by moe_pack_weights */
} moe_layout_t;

/* Problem shape.  T tokens, hidden size d, E global experts, top-k, SwiGLU
 * width F, local expert block [expert_begin, expert_begin + num_local);
 * act / weight hold moe_dtype_t values, weight_layout a moe_layout_t
 * (MOE_LAYOUT_BLOCKED needs BF16, FP8_E4M3 or MXFP4 weights). */
typedef struct {
  int32_t T, d, E, k, F;
  int32_t expert_begin, num_local;
  int32_t act, weight;
  int32_t weight_layout;
} moe_problem_t;

/* Bytes of scratch `call` needs for problem p (0 if p is invalid).  The
 * scratch must be device memory, 256-byte aligned; its contents on entry do
 * not matter and are undefined on return. */
size_t moe_workspace_size(const moe_problem_t* p, int32_t call);

/* Static, human-readable name of a status code. */
const char* moe_status_string(moe_status_t s);

/* Router and gate ("What is an MoE layer?": the gate picks a few experts per
 * token).
 *  x        [T][d] act format.
 *  w_router [d][E] act format, or NULL: then `logits` is an INPUT [T][E]
 *           float32 and only selection and gates run.
 *  router_bias [E] float32 or NULL (zero): added to the logits, so it moves
 *           both the selection and the gate values.
 *  logits   [T][E] float32, required: the output L (including the bias)
 *           when w_router != NULL, the input when w_router == NULL.
 *  topk_idx [T][k] int32 output: global expert ids ordered by (-L, e).
 *           A NaN logit ranks as -inf (it ties with -inf and with other
 *           NaNs, and those ties also go to the lower index), so every row
 *           yields k distinct ids in [0, E).
 *  topk_w   [T][k] float32 output: renormalised gates (sum to 1 per token);
 *           unspecified for a row whose chosen logits are not all finite.
 *  ws, ws_bytes: scratch of moe_workspace_size(p, MOE_CALL_ROUTE) bytes (the
 *           router matrix transposed to [E][d] and K-split partial sums);
 *           may be NULL / 0 when w_router == NULL.
 * The selection is taken on exactly the float32 values written to `logits`. */
moe_status_t moe_route(const moe_problem_t* p, const void* x, const void* w_router,
                       const float* router_bias, float* logits, int32_t* topk_idx,
                       float* topk_w, void* ws, size_t ws_bytes, void* stream);

/* Dispatch order ("Mechanics of Token Routing": tokens go to their expert):
 * a stable counting sort of the slots whose expert is local.
 *  topk_idx    [T*k] int32 input.
 *  counts      [E_l] int32 output: kept slots per local expert.
 *  offsets     [E_l + 1] int32 output: exclusive prefix of counts;
 *              offsets[E_l] = N, the number of kept slots.
 *  sorted_slot [T*k] int32 output: rows 0..N-1 hold the kept slots grouped
 *              by local expert, increasing s inside each group; rows N.. are
 *              left unspecified.
 *  slot_pos    [T*k] int32 output: position of slot s in sorted_slot, or -1
 *              if s is not kept.
 *  ws / ws_bytes: scratch of at least moe_workspace_size(p, MOE_CALL_PERMUTE). */
moe_status_t moe_permute(const moe_problem_t* p, const int32_t* topk_idx, int32_t* counts,
                         int32_t* offsets, int32_t* sorted_slot, int32_t* slot_pos,
                         void* ws, size_t ws_bytes, void* stream);

/* Local experts ("Tensor parallel vs expert parallel": full-size expert
 * GEMMs on the dispatched tokens): for every kept row p < offsets[E_l], with
 * s = sorted_slot[p], t = s / k and j the local expert whose segment
 * [offsets[j], offsets[j+1]) holds p:
 *    y[p] = FFN_{expert_begin + j}(x[t]) * (topk_w ? topk_w[s] : 1)
 *  x           [T][d] act format.
 *  sorted_slot [T*k], offsets [E_l + 1]: as produced by moe_permute.
 *  w_gate, w_up [E_l][F][d], w_down [E_l][d][F] in the weight format.
 *  s_gate, s_up, s_down: block scales (required for FP8_E4M3 and MXFP4, in
 *              the layouts above; else ignored).
 *  topk_w      [T*k] float32 gates or NULL (y left unweighted).
 *  y           [T*k][d] act format output; rows >= N are not written.
 *  ws / ws_bytes: scratch of at least moe_workspace_size(p, MOE_CALL_EXPERT_FFN). */
moe_status_t moe_expert_ffn(const moe_problem_t* p, const void* x, const int32_t* sorted_slot,
                            const int32_t* offsets, const void* w_gate, const void* w_up,
                            const void* w_down, const void* s_gate, const void* s_up,
                            const void* s_down, const float* topk_w, void* y, void* ws,
                            size_t ws_bytes, void* stream);

/* Combine ("Mechanics of Token Routing": the output travels back), without
 * atomics, in a fixed order:
 *    out[t] = sum_{i = 0..k-1, slot_pos[t*k+i] >= 0} y[slot_pos[t*k+i]] * (topk_w ? topk_w[t*k+i] : 1)
 * accumulated in float32 in increasing i and rounded once to the act format;
 * a token with no kept slot gets 0.
 *  y [T*k][d] act format; slot_pos [T*k]; topk_w [T*k] float32 or NULL
 *  (y already weighted); out [T][d] act format output. */
moe_status_t moe_combine(const moe_problem_t* p, const void* y, const int32_t* slot_pos,
                         const float* topk_w, void* out, void* stream);

/* Arguments of moe_forward.  Required: x, w_gate, w_up, w_down, out, and
 * either w_router, or logits as an input.  s_* are required for FP8 and MXFP4 weights.
 * The remaining outputs are optional (NULL = not wanted) and hold what the
 * individual calls above would write. */
typedef struct {
  const void* x;            /* [T][d] act */
  const void* w_router;     /* [d][E] act, or NULL (logits is then an input) */
  const float* router_bias; /* [E] or NULL */
  const void* w_gate;       /* [E_l][F][d] weight format */
  const void* w_up;         /* [E_l][F][d] */
  const void* w_down;       /* [E_l][d][F] */
  const void* s_gate;       /* FP8 / MXFP4 block scales, see above */
  const void* s_up;
  const void* s_down;
  void* out;                /* [T][d] act output */
  float* logits;            /* [T][E] output (or input when w_router == NULL) */
  int32_t* topk_idx;        /* [T][k] */
  float* topk_w;            /* [T][k] */
  int32_t* counts;          /* [E_l] */
  int32_t* offsets;         /* [E_l + 1] */
  int32_t* sorted_slot;     /* [T*k] */
  int32_t* slot_pos;        /* [T*k] */
  /* Optional stage timing: NULL, or MOE_FORWARD_EVENTS hipEvent_t handles
   * (created by the caller, passed as void*) that moe_forward records on
   * `stream` at the stage boundaries: [0] before the router, [1] after the
   * router, [2] after the permutation, [3] after the expert tile schedule,
   * [4] after the gate/up GEMM, [5] after the down GEMM, [6] after the
   * combine.  A failed record returns MOE_ERR_HIP. */
  void* const* events;
} moe_forward_args_t;

#define MOE_FORWARD_EVENTS 7

/* The whole layer ("Expert Parallelism for MoE Models" (apxml), section
 * "Mechanics of Token Routing and All-to-All Communication": route each token
 * to its experts, let each expert compute, send the outputs back and sum
 * them): route, permute, expert FFN (gates folded into the down projection's
 * epilogue), combine, with the results of the individual calls above.  No
 * host synchronisation: the data-dependent sizes (counts, N) never return to
 * the host.
 *  ws / ws_bytes: scratch of at least moe_workspace_size(p, MOE_CALL_FORWARD). */
moe_status_t moe_forward(const moe_problem_t* p, const moe_forward_args_t* a, void* ws,
                         size_t ws_bytes, void* stream);

/* ---- The whole layer without caller scratch ----
 *
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * moe_forward with its scratch in a device array that the library holds,
 * MOE_NOALLOC_SCRATCH_BYTES bytes on every GPU it runs on, from the first
 * call on that GPU until the process ends.  Same arguments, kernels and
 * results as moe_forward; the caller still passes every input and output.
 * Nothing is allocated or freed by the call.
 *  - Problems whose moe_workspace_size(p, MOE_CALL_FORWARD) exceeds
 *    MOE_NOALLOC_SCRATCH_BYTES return MOE_ERR_UNSUPPORTED (64 MiB holds, for
 *    instance, the Qwen3-30B-A3B shape up to 1023 tokens, its decode-sized
 *    tile plans; from 64 slots per expert the prefill-sized plans add 64 MiB
 *    of tail partial sums); invalid problems return moe_forward's status.
 *  - All calls on one GPU share that GPU's array, which keeps the last call's
 *    contents (no call relies on them): calls that overlap in time on one
 *    GPU, from several streams or host threads, race on it and must be
 *    serialised by the caller (one stream does that).
 *  - The first call on a GPU looks the array's device address up (a HIP
 *    runtime query, no allocation); a failure there returns MOE_ERR_HIP. */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)

moe_status_t moe_forward_noalloc(const moe_problem_t* p, const moe_forward_args_t* a,
                                 void* stream);

/* ---- Expert-parallel load balancing (EPLB) ----
 *
 * "Serving MoE models with expert parallelism on 8xH200" (reviosa), section
 * "Routing imbalance": per-expert token counts measure the load; the busiest
 * GPU's count over the mean is the imbalance factor; hot experts get
 * redundant copies placed on less-loaded GPUs, and co-locating hot with cold
 * experts evens the load without copies.  The pages give no algorithm; the
 * one here (host code, deterministic):
 *  1. copies: P = E + R physical slots on G ranks, S = P / G per rank; each
 *     of the R spare slots in turn goes to the expert with the largest load
 *     per copy, load[e] / replicas[e] (exact comparison, ties to the lower
 *     id), among experts with fewer than G copies;
 *  2. placement: each copy carries load[e] / replicas[e] (double); copies,
 *     heaviest first (ties: lower expert id, then lower copy index), go to
 *     the least-loaded rank (double sum of its copies in placement order;
 *     ties to the lower rank) among ranks with a free slot that hold no copy
 *     of the same expert (if there is none, among ranks with a free slot);
 *  3. numbering: rank g owns physical ids g*S .. g*S + S - 1, holding its
 *     experts in increasing id; copy j of expert e is the j-th smallest
 *     physical id holding e.
 * A rank then runs moe_permute / moe_expert_ffn / moe_combine with E = P,
 * expert_begin = g*S, num_local = S, on the ids moe_eplb_remap writes and on
 * its physical slots' weights (copies of the logical experts' weights).  The
 * ranks' outputs add up to the layer's output for any plan.
 *
 * moe_eplb_plan - host function (host pointers, nothing enqueued).
 *  load         [E] int64, tokens routed to each expert over the caller's
 *               window (e.g. sums of moe_permute's counts), 0 <= load < 2^40
 *  replicas     [E] int32 output, copies per expert (1 .. G)
 *  phys_to_log  [E + R] int32 output, logical expert of each physical slot
 *  log_to_phys  [E][G] int32 output, physical slot of copy j of expert e
 *               (j < replicas[e]), -1 beyond
 *  rank_load    [G] double output or NULL, the planned load per rank
 * Limits: 1 <= E, 1 <= G, 0 <= R <= E*(G-1), (E + R) divisible by G,
 * E + R <= 512.  Otherwise MOE_ERR_INVALID_ARGUMENT (MOE_ERR_UNSUPPORTED for
 * E + R > 512), with the outputs untouched. */
moe_status_t moe_eplb_plan(const int64_t* load, int32_t E, int32_t G, int32_t R,
                           int32_t* replicas, int32_t* phys_to_log, int32_t* log_to_phys,
                           double* rank_load);

/* moe_eplb_remap - device: logical top-k ids -> physical ids.  The slot of
 * token t routed to expert e goes to copy (t mod replicas[e]):
 *   topk_phys[t*k + i] = log_to_phys[e*G + t % replicas[e]],  e = topk_idx[t*k + i]
 * and -1 (never local on any rank) for e outside [0, E) or a replicas entry
 * outside [1, G].
 *  topk_idx [T*k], replicas [E], log_to_phys [E*G], topk_phys [T*k]: device
 *  arrays (topk_phys may not alias the others).  Limits: T >= 0, 1 <= k,
 *  T*k < 2^31, 1 <= E, 1 <= G, E*G < 2^31. */
moe_status_t moe_eplb_remap(int32_t T, int32_t k, int32_t E, int32_t G, const int32_t* topk_idx,
                            const int32_t* replicas, const int32_t* log_to_phys,
                            int32_t* topk_phys, void* stream);

/* Blocked weight layout (for callers that convert weights once at load
 * time): each expert matrix [Nout][K] is stored as [Nout/32][K/64] units of
 * 32 rows x 64 K values.  A unit is the sequence of 1 KB MFMA operand loads
 * of one wave for that block (load q, lane l: 16 bytes of row
 * 32*block + feat(l % 32), the bytes of K chunk 2q + l/32 of the unit, feat
 * the GEMMs' permuted feature order inside a 32-row block), so a stage of a
 * weight block streams as one contiguous run, and a wave's operand load, from
 * LDS or straight from memory, is 1 KB contiguous.  Same size as the
 * row-major matrix; the scales keep their layouts.  Results equal those of
 * the row-major layout bit for bit, except in the decode-sized plans (at
 * most 64 slots per local expert with bf16 or MXFP4 weights), which sum the
 * K products in another order on the two layouts (within the same
 * tolerances).
 *  which: 0 = a gate or up matrix set [E_l][F][d] (call once for each),
 *         1 = the down matrix set [E_l][d][F].
 *  src, dst: device arrays of the matrix set's size (distinct).  The weight
 *  format is p->weight (BF16, FP8_E4M3 or MXFP4); p->weight_layout is
 *  ignored. */
moe_status_t moe_pack_weights(const moe_problem_t* p, int32_t which, const void* src, void* dst,
                              void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
