// Dispatch order: a stable counting sort of the kept slots by local expert.
//
// "Expert Parallelism for MoE Models" (apxml), section "Mechanics of Token
// Routing and All-to-All Communication": each token is sent to the device
// that hosts its expert.  On one device that is a gather into expert-sorted
// order.  The sort has one correct result: the slots of each local expert in
// increasing slot index s = t*k + i.
//
// Three kernels, none with an order-dependent atomic:
//   1. hist:    each workgroup counts the kept slots of its 2048-slot chunk per
//               local expert (LDS counters; counting is order-free).
//   2. scan:    one workgroup sums the chunk counts per expert, scans them into
//               `offsets`, turns the chunk counts into each chunk's first
//               position inside every expert segment, and writes the expert
//               GEMM's tile schedule.
//   3. scatter: each workgroup walks its chunk in slot order, 256 slots per
//               round; a slot's rank among equal experts inside its wave comes
//               from ballots over the expert id bits, across waves from
//               per-wave counts in LDS, across rounds from a running base.
// A decode batch has few slots (T*k <= 8192): then one workgroup of 16 waves
// runs all three phases in one kernel, and also writes the expert GEMM's tile
// schedule (the M tiles of every expert segment), saving four launches.
#include "dispatch_sort.h"
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kChunk = kPermuteChunk;   // slots per workgroup
constexpr int kThreads = 256;
constexpr int kRounds = kChunk / kThreads;

__global__ __launch_bounds__(kThreads) void permute_hist_kernel(const int32_t* __restrict__ idx,
                                                                long long S, int e0, int El,
                                                                int nb, int32_t* blk_cnt) {
  __shared__ int hist[kMaxExperts];
  const int b = blockIdx.x;
  for (int e = threadIdx.x; e < El; e += kThreads) hist[e] = 0;
  __syncthreads();
  const long long base = (long long)b * kChunk;
  for (int r = 0; r < kRounds; ++r) {
    const long long s = base + r * kThreads + threadIdx.x;
    if (s < S) {
      const int e = idx[s] - e0;
      if ((unsigned)e < (unsigned)El) atomicAdd(&hist[e], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < El; e += kThreads) blk_cnt[(size_t)e * nb + b] = hist[e];
}

// One workgroup of kMaxExperts threads: thread e owns local expert e.  The
// chunk counts are staged through LDS with coalesced loads and stores when
// they fit (rows padded by one word against bank conflicts).  With `tiles`,
// it also writes the expert GEMM's tile schedule (the M tiles of every expert
// segment), which saves the schedule kernel.
constexpr int kScanLds = 12288;  // staged counts (48 KB)

__global__ __launch_bounds__(kMaxExperts) void permute_scan_kernel(int El, int nb, int32_t* blk,
                                                                   int32_t* counts,
                                                                   int32_t* offsets, int bm,
                                                                   int4* tiles, int* ntiles) {
  __shared__ long long wave_tot[kMaxExperts / kWave];
  __shared__ int stage[kScanLds];
  const int e = threadIdx.x;
  const int pitch = nb + 1;
  const bool staged = (long long)El * pitch <= kScanLds;
  if (staged) {
    for (int i = e; i < El * nb; i += kMaxExperts) stage[(i / nb) * pitch + i % nb] = blk[i];
    __syncthreads();
  }
  auto at = [&](int b) -> int& { return staged ? stage[e * pitch + b] : blk[(size_t)e * nb + b]; };
  int cnt = 0;
  if (e < El)
    for (int b = 0; b < nb; ++b) cnt += at(b);
  const int nt = (tiles && e < El) ? (cnt + bm - 1) / bm : 0;
  // inclusive scans over the experts of the slots (low 32 bits) and the M
  // tiles (high 32 bits): both totals stay below 2^31
  const long long both = block_inclusive_scan<kMaxExperts>(
      (long long)cnt | ((long long)nt << 32), wave_tot);
  const int incl_s = (int)(both & 0xffffffffLL), incl_t = (int)(both >> 32);
  const int excl = incl_s - cnt;
  if (e < El) {
    counts[e] = cnt;
    offsets[e] = excl;
    int run = excl;
    for (int b = 0; b < nb; ++b) {
      const int c = at(b);
      at(b) = run;
      run += c;
    }
    const int tfirst = incl_t - nt;
    for (int i = 0; i < nt; ++i) tiles[tfirst + i] = make_int4(e, excl + i * bm, excl + cnt, 0);
  }
  if (e == El - 1) {
    offsets[El] = incl_s;
    if (tiles) *ntiles = incl_t;
  }
  if (staged) {
    __syncthreads();
    for (int i = e; i < El * nb; i += kMaxExperts) blk[i] = stage[(i / nb) * pitch + i % nb];
  }
}

__global__ __launch_bounds__(kThreads) void permute_scatter_kernel(
    const int32_t* __restrict__ idx, long long S, int e0, int El, int nbits, int nb,
    const int32_t* __restrict__ blk_off, int32_t* sorted_slot, int32_t* slot_pos) {
  __shared__ int base[kMaxExperts];
  __shared__ int wcnt[kThreads / kWave][kMaxExperts];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int w = tid / kWave;
  const int l = lane_id();
  for (int e = tid; e < El; e += kThreads) {
    base[e] = blk_off[(size_t)e * nb + b];
#pragma unroll
    for (int q = 0; q < kThreads / kWave; ++q) wcnt[q][e] = 0;
  }
  __syncthreads();
  const unsigned long long below = (1ull << l) - 1ull;
  for (int r = 0; r < kRounds; ++r) {
    const long long s = (long long)b * kChunk + r * kThreads + tid;
    const bool valid = s < S;
    int e = valid ? idx[s] - e0 : -1;
    const bool keep = valid && (unsigned)e < (unsigned)El;
    if (valid && !keep) slot_pos[s] = -1;
    // lanes of this wave holding the same local expert
    unsigned long long m = __ballot(keep);
    for (int bit = 0; bit < nbits; ++bit) {
      const bool on = keep && ((e >> bit) & 1);
      const unsigned long long v = __ballot(on);
      m &= on ? v : ~v;
    }
    const int rank = __popcll(m & below);
    const int cnt = __popcll(m);
    if (keep && rank == 0) wcnt[w][e] = cnt;
    __syncthreads();
    if (keep) {
      int pos = base[e] + rank;
      for (int q = 0; q < w; ++q) pos += wcnt[q][e];
      sorted_slot[pos] = (int32_t)s;
      slot_pos[s] = pos;
    }
    __syncthreads();
    if (keep && rank == 0) {
      atomicAdd(&base[e], cnt);  // a sum: the result does not depend on order
      wcnt[w][e] = 0;
    }
    __syncthreads();
  }
}

constexpr int kSmallThreads = 1024;
constexpr long long kSmallSlots = 8192;

__global__ __launch_bounds__(kSmallThreads) void permute_small_kernel(
    const int32_t* __restrict__ idx, int S, int e0, int El, int nbits, int32_t* counts,
    int32_t* offsets, int32_t* sorted_slot, int32_t* slot_pos, int bm, int4* tiles, int* ntiles) {
  __shared__ DispatchSortLds<kSmallThreads> sm;
  dispatch_sort<kSmallThreads>(idx, S, e0, El, nbits, counts, offsets, sorted_slot, slot_pos, bm,
                               tiles, ntiles, sm);
}

}  // namespace

size_t permute_ws_bytes(const Shape& s) {
  const long long nb = (s.S + kChunk - 1) / kChunk;
  return align_up((size_t)nb * s.El * sizeof(int32_t));
}

hipError_t permute(const Shape& s, const int32_t* topk_idx, int32_t* counts, int32_t* offsets,
                   int32_t* sorted_slot, int32_t* slot_pos, void* ws, hipStream_t st,
                   const FfnSchedule* sched, bool* sched_written) {
  if (sched_written) *sched_written = false;
  int nbits = 0;
  while ((1 << nbits) < s.El) ++nbits;
  if (s.S <= kSmallSlots) {
    hipLaunchKernelGGL(permute_small_kernel, dim3(1), dim3(kSmallThreads), 0, st, topk_idx,
                       (int)s.S, s.e0, s.El, nbits, counts, offsets, sorted_slot, slot_pos,
                       sched ? sched->bm : 1, sched ? sched->tiles : nullptr,
                       sched ? sched->ntiles : nullptr);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess && sched_written) *sched_written = sched != nullptr;
    return e;
  }
  const int nb = (int)((s.S + kChunk - 1) / kChunk);
  int32_t* blk = static_cast<int32_t*>(ws);
  if (nb > 0) {
    hipLaunchKernelGGL(permute_hist_kernel, dim3(nb), dim3(kThreads), 0, st, topk_idx, s.S, s.e0,
                       s.El, nb, blk);
  }
  hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(kMaxExperts), 0, st, s.El, nb, blk, counts,
                     offsets, sched ? sched->bm : 1, sched ? sched->tiles : nullptr,
                     sched ? sched->ntiles : nullptr);
  if (nb > 0) {
    hipLaunchKernelGGL(permute_scatter_kernel, dim3(nb), dim3(kThreads), 0, st, topk_idx, s.S,
                       s.e0, s.El, nbits, nb, blk, sorted_slot, slot_pos);
  }
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && sched_written) *sched_written = sched != nullptr;
  return e;
}

}  // namespace moe
