// Combine: gate-weighted sum of each token's expert outputs, back in token
// order, without atomics.
//
// "Expert Parallelism for MoE Models" (apxml), section "Mechanics of Token
// Routing and All-to-All Communication": after the expert computes, its output
// is sent back to the token.  out[t] = sum over i of the kept slots t*k + i of
// y[slot_pos[t*k + i]] (times the gate when y is unweighted), accumulated in
// float32 in increasing i and rounded once.  A token with no kept slot gets 0.
//
// One workgroup per token row; each thread owns 8 consecutive columns (one
// 16-byte bf16 chunk, or two 16-byte float32 chunks), so every y row is read
// with full-width coalesced loads.  With k <= 8 a token's slot positions and
// gates are loaded once for all its columns, and a token without a local slot
// only writes zeros.  The pass is HBM-bound; bf16 rows are read and written
// with nontemporal accesses (each byte is touched once: measured 55 -> 48 us
// on the Qwen3 prefill's 268 MB of expert outputs).
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kMaxThreads = 256;  // 8 columns per thread; 256 or 128 threads

// Accumulate the rows of slots t*k + i0 .. + kBatch - 1 (those with pos >= 0)
// into acc, in increasing i; every row load of the batch is issued first.
template <bool kBF16, int kBatch>
__device__ __forceinline__ void combine_batch(const void* y, const int* pos, const float* gw,
                                              int d, int c0, float* acc) {
  u32x4_t raw[kBatch][kBF16 ? 1 : 2];
#pragma unroll
  for (int b = 0; b < kBatch; ++b) {
    if (pos[b] < 0) continue;
    if constexpr (kBF16) {
      raw[b][0] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(
          static_cast<const uint16_t*>(y) + (long long)pos[b] * d + c0));
    } else {
      const float* yr = static_cast<const float*>(y) + (long long)pos[b] * d + c0;
      raw[b][0] = *reinterpret_cast<const u32x4_t*>(yr);
      raw[b][1] = *reinterpret_cast<const u32x4_t*>(yr + 4);
    }
  }
#pragma unroll
  for (int b = 0; b < kBatch; ++b) {
    if (pos[b] < 0) continue;
    if constexpr (kBF16) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t u = raw[b][0][q];
        acc[2 * q] = fmaf(bf16_to_f32(uint16_t(u & 0xffff)), gw[b], acc[2 * q]);
        acc[2 * q + 1] = fmaf(bf16_to_f32(uint16_t(u >> 16)), gw[b], acc[2 * q + 1]);
      }
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] = fmaf(__uint_as_float(raw[b][q >> 2][q & 3]), gw[b], acc[q]);
    }
  }
}

template <bool kBF16>
__device__ __forceinline__ void combine_store(void* out, long long t, int d, int c0,
                                              const float* acc) {
  if constexpr (kBF16) {
    __builtin_nontemporal_store(
        u32x4_t{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])},
        reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(out) + t * d + c0));
  } else {
    float* orow = static_cast<float*>(out) + t * d + c0;
    *reinterpret_cast<f32x4_t*>(orow) = f32x4_t{acc[0], acc[1], acc[2], acc[3]};
    *reinterpret_cast<f32x4_t*>(orow + 4) = f32x4_t{acc[4], acc[5], acc[6], acc[7]};
  }
}

template <bool kBF16>
__global__ __launch_bounds__(kMaxThreads) void combine_kernel(const void* y, const int32_t* slot_pos,
                                                           const float* topk_w, void* out, int d,
                                                           int k) {
  const long long t = blockIdx.x;
  constexpr int kBatch = 8;  // slots whose rows are loaded together
  if (k <= kBatch) {
    // the token's slot positions and gates, loaded once for all its columns
    int pos[kBatch];
    float gw[kBatch];
    bool any = false;
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      pos[b] = b < k ? slot_pos[t * k + b] : -1;
      gw[b] = (b < k && topk_w) ? topk_w[t * k + b] : 1.0f;
      any = any || pos[b] >= 0;
    }
    for (int c0 = threadIdx.x * 8; c0 < d; c0 += blockDim.x * 8) {
      float acc[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] = 0.f;
      if (any) combine_batch<kBF16, kBatch>(y, pos, gw, d, c0, acc);
      combine_store<kBF16>(out, t, d, c0, acc);
    }
    return;
  }
  for (int c0 = threadIdx.x * 8; c0 < d; c0 += blockDim.x * 8) {
    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = 0.f;
    for (int i0 = 0; i0 < k; i0 += kBatch) {
      int pos[kBatch];
      float gw[kBatch];
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        const long long s = t * k + i0 + b;
        pos[b] = i0 + b < k ? slot_pos[s] : -1;
        gw[b] = (i0 + b < k && topk_w) ? topk_w[s] : 1.0f;
      }
      combine_batch<kBF16, kBatch>(y, pos, gw, d, c0, acc);
    }
    combine_store<kBF16>(out, t, d, c0, acc);
  }
}

}  // namespace

hipError_t combine(const Shape& s, const void* y, const int32_t* slot_pos, const float* topk_w,
                   void* out, hipStream_t st) {
  if (s.T == 0) return hipSuccess;
  // whole passes over the row: 256 threads when d is a multiple of 2048, else
  // 128 (d / 8 is a multiple of 16)
  const int threads = (s.d % 2048) == 0 ? 256 : 128;
  if (s.act == kBF16)
    hipLaunchKernelGGL(combine_kernel<true>, dim3(s.T), dim3(threads), 0, st, y, slot_pos, topk_w,
                       out, s.d, s.k);
  else
    hipLaunchKernelGGL(combine_kernel<false>, dim3(s.T), dim3(threads), 0, st, y, slot_pos,
                       topk_w, out, s.d, s.k);
  return hipGetLastError();
}

}  // namespace moe
