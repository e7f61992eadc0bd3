// The dispatch order of a small batch, computed by one workgroup: a stable
// counting sort of the kept slots by local expert, plus the expert GEMMs'
// tile schedule, as a device routine any one-workgroup kernel can run (the
// permutation kernel for small batches does).
//
// "Expert Parallelism for MoE Models" (apxml), section "Mechanics of Token
// Routing and All-to-All Communication": each token is sent to the device
// that hosts its expert; on one device that is a gather into expert-sorted
// order.  The sort has one correct result: the slots of each local expert in
// increasing slot index s = t*k + i.
#pragma once

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

// Inclusive prefix sum over the kThreads threads of a workgroup (thread
// order): a shuffle scan inside each wave, then each wave adds the totals of
// the waves before it (two barriers instead of one per doubling step).
// Integer sums, so the result does not depend on the order of additions.
// `wave_tot`: LDS scratch of kThreads / 64 elements.
template <int kThreads, typename V>
__device__ __forceinline__ V block_inclusive_scan(V v, V* wave_tot) {
  const int l = lane_id();
  const int w = threadIdx.x / kWave;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const V t = __shfl_up(v, o, kWave);
    if (l >= o) v += t;
  }
  if (l == kWave - 1) wave_tot[w] = v;
  __syncthreads();
  V add = 0;
  for (int q = 0; q < w; ++q) add += wave_tot[q];
  __syncthreads();  // wave_tot may be reused by the caller
  return v + add;
}

// LDS a workgroup of kThreads threads needs for dispatch_sort.
template <int kThreads>
struct DispatchSortLds {
  int hist[kMaxExperts];
  int base[kMaxExperts];
  int wave_tot[kThreads / kWave];
  int wcnt[kThreads / kWave][kMaxExperts];
};

// One workgroup of kThreads threads (kThreads >= El): counts, offsets,
// sorted_slot and slot_pos of the S <= 8192 slots whose expert ids are in
// idx (global or LDS), and, with `tiles`, the M tiles of bm rows of every
// expert segment.  Ids outside [e0, e0 + El) are not local (slot_pos -1).
// Every thread of the workgroup must call it.
template <int kThreads>
__device__ void dispatch_sort(const int32_t* idx, int S, int e0, int El, int nbits,
                              int32_t* counts, int32_t* offsets, int32_t* sorted_slot,
                              int32_t* slot_pos, int bm, int4* tiles, int* ntiles,
                              DispatchSortLds<kThreads>& sm) {
  static_assert(kThreads >= kMaxExperts, "a thread per local expert in the scan");
  constexpr int kWaves = kThreads / kWave;
  const int tid = threadIdx.x;
  const int w = tid / kWave;
  const int l = lane_id();
  for (int e = tid; e < El; e += kThreads) {
    sm.hist[e] = 0;
#pragma unroll
    for (int q = 0; q < kWaves; ++q) sm.wcnt[q][e] = 0;
  }
  __syncthreads();
  for (int s = tid; s < S; s += kThreads) {
    const int e = idx[s] - e0;
    if ((unsigned)e < (unsigned)El) atomicAdd(&sm.hist[e], 1);
  }
  __syncthreads();
  // exclusive scan of the counts (and of the M tiles per expert)
  const int cnt = tid < El ? sm.hist[tid] : 0;
  const int nt = (cnt + bm - 1) / bm;
  // both sums fit 16 bits: at most 8192 slots and 8192 + El tiles
  const int incl = block_inclusive_scan<kThreads>(cnt | (nt << 16), sm.wave_tot);
  const int off = (incl & 0xffff) - cnt;
  const int tfirst = (incl >> 16) - nt;
  if (tid < El) {
    counts[tid] = cnt;
    offsets[tid] = off;
    sm.base[tid] = off;
    if (tiles)
      for (int i = 0; i < nt; ++i) tiles[tfirst + i] = make_int4(tid, off + i * bm, off + cnt, 0);
  }
  if (tid == El - 1) {
    offsets[El] = incl & 0xffff;
    if (tiles) *ntiles = incl >> 16;
  }
  __syncthreads();
  // stable scatter, kThreads slots per round in slot order: a slot's rank
  // among the equal experts of its wave from ballots over the expert id bits,
  // across waves from per-wave counts, across rounds from a running base
  const unsigned long long below = (1ull << l) - 1ull;
  for (int r0 = 0; r0 < S; r0 += kThreads) {
    const int s = r0 + tid;
    const bool valid = s < S;
    const int e = valid ? idx[s] - e0 : -1;
    const bool keep = valid && (unsigned)e < (unsigned)El;
    if (valid && !keep) slot_pos[s] = -1;
    unsigned long long m = __ballot(keep);
    for (int bit = 0; bit < nbits; ++bit) {
      const bool on = keep && ((e >> bit) & 1);
      const unsigned long long v = __ballot(on);
      m &= on ? v : ~v;
    }
    const int rank = __popcll(m & below);
    const int c = __popcll(m);
    if (keep && rank == 0) sm.wcnt[w][e] = c;
    __syncthreads();
    if (keep) {
      int pos = sm.base[e] + rank;
      for (int q = 0; q < w; ++q) pos += sm.wcnt[q][e];
      sorted_slot[pos] = s;
      slot_pos[s] = pos;
    }
    __syncthreads();
    if (keep && rank == 0) {
      atomicAdd(&sm.base[e], c);  // a sum: the result does not depend on order
      sm.wcnt[w][e] = 0;
    }
    __syncthreads();
  }
}

}  // namespace moe
