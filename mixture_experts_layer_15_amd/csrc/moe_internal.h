// Internal host-side interface between the C ABI (moe_api.cpp) and the
// kernel launchers (*.hip).  Not installed; callers use include/moe.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

namespace moe {

enum Fmt : int { kF32 = 0, kBF16 = 1, kFP8 = 2, kFP4 = 3 };

constexpr int kMaxExperts = 512;      // E limit (router top-k and permutation LDS tables)
constexpr int kPermuteChunk = 2048;   // slots per workgroup in the permutation kernels

// Validated problem shape.  S = T*k slots.
struct Shape {
  int T, d, E, k, F, e0, El;
  int act, weight;
  int blocked;  // expert weights in the blocked layout of pack_weights
  long long S;
};

inline size_t align_up(size_t v, size_t a = 256) { return (v + a - 1) / a * a; }

// hipFuncSetAttribute for the dynamic LDS size of `kern`, once per device
// (devices 0..63 remembered in an atomic bit set; the call is idempotent, so
// two threads that both make it race harmlessly).
inline hipError_t set_lds_attr(const void* kern, int bytes, std::atomic<uint64_t>& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? (uint64_t)1 << dev : 0;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_release);
  return e;
}
inline int act_bytes(const Shape& s) { return s.act == kF32 ? 4 : 2; }

// ---- route.hip
// K splits of the router GEMM used by moe_forward, and the scratch they need.
int router_splits(const Shape& s);
size_t route_ws_bytes(const Shape& s);
// w_router != null: logits = x W_r + bias are published to `logits` and
// selected on; scratch holds route_ws_bytes (the transposed router matrix and
// K-split partials).  w_router == null: `logits_in` holds the final logits
// (scratch may be null).
hipError_t route(const Shape& s, const void* x, const void* w_router, const float* bias,
                 const float* logits_in, float* logits, int32_t* topk_idx, float* topk_w,
                 void* scratch, hipStream_t st);
bool use_router_gemm(const Shape& s);

// prod [ks][T][E] = x W_r (float32 accumulation, K cut into
// ks = router_gemm_splits(s) parts, one plane each) from the router matrix
// stored [E][d]
int router_gemm_splits(const Shape& s);
hipError_t router_gemm(const Shape& s, const void* x, const void* w_router_t, float* prod,
                       hipStream_t st);

// ---- ffn.hip (tile schedule shared with the permutation)
struct FfnSchedule {
  int4* tiles;   // (local expert, first row, expert's end row, 0) of every M tile
  int* ntiles;   // number of M tiles
  int bm;        // M tile height
};
FfnSchedule ffn_schedule_view(const Shape& s, void* ffn_ws);
size_t ffn_ws_bytes(const Shape& s);
// schedule_ready: the tile schedule in ffn_ws was already written (by the
// permutation); stage_events: null or 3 events recorded after the schedule,
// the gate/up GEMM and the down GEMM.
hipError_t expert_ffn(const Shape& s, const void* x, const int32_t* sorted_slot,
                      const int32_t* offsets, const void* w_gate, const void* w_up,
                      const void* w_down, const void* s_gate, const void* s_up,
                      const void* s_down, const float* topk_w, void* y, void* ws,
                      hipStream_t st, bool schedule_ready = false,
                      hipEvent_t const* stage_events = nullptr);

// ---- permute.hip
size_t permute_ws_bytes(const Shape& s);
// When `sched` is non-null and the single-workgroup path runs, the expert
// tile schedule is written too and *sched_written is set.
hipError_t permute(const Shape& s, const int32_t* topk_idx, int32_t* counts, int32_t* offsets,
                   int32_t* sorted_slot, int32_t* slot_pos, void* ws, hipStream_t st,
                   const FfnSchedule* sched = nullptr, bool* sched_written = nullptr);

// ---- combine.hip
hipError_t combine(const Shape& s, const void* y, const int32_t* slot_pos, const float* topk_w,
                   void* out, hipStream_t st);

// Blocked layout of one stored expert weight matrix [Nout][K] (any weight
// format but float32): [Nout/32][K/64][32 rows][64 K values], each 32 x 64
// unit being the LDS image the expert GEMMs stage for that block (rows in
// the MFMA feature order, 16-byte chunks XOR-swizzled).  Same size as the
// row-major matrix.
hipError_t pack_weights(const Shape& s, int which, const void* src, void* dst, hipStream_t st);

// ---- eplb.hip
// The placement plan of moe_eplb_plan (arguments already checked).
int eplb_plan(const int64_t* load, int E, int G, int R, int32_t* replicas, int32_t* phys_to_log,
              int32_t* log_to_phys, double* rank_load);
hipError_t eplb_remap(int T, int k, int E, int G, const int32_t* topk_idx,
                      const int32_t* replicas, const int32_t* log_to_phys, int32_t* topk_phys,
                      hipStream_t st);

}  // namespace moe
