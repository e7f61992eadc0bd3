// Router logits and softmax top-k gating on gfx950.
//
// "Wide Expert Parallelism" (llm-d notes), section "What is an MoE layer?":
// a small gate inspects every token and sends it to a few of the experts.
// Here: L = x W_r + b with float32 accumulation, the k largest L per token
// ordered by (-L, e) (ties to the lower expert index), and gates equal to a
// softmax over the k chosen logits (a softmax over all E renormalised over
// the chosen k: the full denominator cancels).
//
// One workgroup owns 32 tokens and every expert column.  bf16: the router
// GEMM runs on MFMA 32x32x16 with the K dimension split four ways across the
// waves (each wave streams a quarter of W_r, staged through LDS in its natural
// [k][e] layout), and the four partial tiles are added in a fixed order.  The
// float32 logits of the tile stay in LDS, so selection and gates happen in the
// same kernel on exactly the values written to `logits`.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kBM = 32;        // tokens per workgroup
constexpr int kCC = 128;       // expert columns per pass (4 MFMA blocks of 32)
constexpr int kBK = 32;        // K rows of W_r per wave per step
constexpr int kThreads = 256;  // 4 waves
constexpr int kStageStride = kCC + 8;  // bf16 elements per staged W_r row (padded)

struct RouteArgs {
  const void* x;         // [T][d]
  const void* w_router;  // [d][E] or null
  const float* bias;     // [E] or null
  const float* logits_in;  // [T][E] (when w_router is null)
  float* logits_out;     // [T][E] or null
  int32_t* topk_idx;     // [T][k]
  float* topk_w;         // [T][k]
  int T, d, E, k;
};

// LDS: a 64 KB region that holds the W_r staging tiles during the K loop and
// the four partial tiles afterwards, then the [32][E] float32 logit tile.
constexpr int kRegionBytes = 4 * kBM * kCC * 4;  // 64 KB

// bf16 router GEMM for one 128-column pass; leaves the finished logits of
// columns [c0, c0 + 128) in lg[r][c].
__device__ void router_pass_bf16(const RouteArgs& a, int t0, int c0, unsigned char* region,
                                 float* lg, int lgs) {
  const int tid = threadIdx.x;
  const int w = tid / kWave;
  const int l = lane_id();
  const uint16_t* x = static_cast<const uint16_t*>(a.x);
  const uint16_t* wr = static_cast<const uint16_t*>(a.w_router);
  uint16_t* stage = reinterpret_cast<uint16_t*>(region) + w * kBK * kStageStride;

  f32x16_t acc[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) acc[b] = f32x16_t{};

  // A operand rows: lane l serves token row l % 32 (clamped to T-1).
  const int arow = min(t0 + (l & 31), a.T - 1);
  const uint16_t* xrow = x + (size_t)arow * a.d;
  const int kgrp = (l >> 5) * 8;  // which 8 of the 16 K values this lane holds

  const int nks = a.d / kBK;
  for (int ks0 = 0; ks0 < nks; ks0 += 4) {
    const int ks = ks0 + w;
    const bool active = ks < nks;
    __syncthreads();  // previous step's readers are done with the staging tile
    if (active) {
      // Stage W_r[k0 .. k0+32)[c0 .. c0+128) : 32 rows x 256 bytes; lane l copies
      // 16 bytes of row (l / 16) + 4 i, columns 8 (l % 16) .. +8.
      const int k0 = ks * kBK;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = (l >> 4) + 4 * i;
        const int c = (l & 15) * 8;
        const uint16_t* src = wr + (size_t)(k0 + r) * a.E + c0 + c;
        uint16_t* dst = stage + r * kStageStride + c;
        if ((a.E & 7) == 0 && c0 + c + 8 <= a.E) {
          *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) dst[j] = (c0 + c + j < a.E) ? src[j] : uint16_t(0);
        }
      }
    }
    __syncthreads();
    if (active) {
      const int k0 = ks * kBK;
#pragma unroll
      for (int kk = 0; kk < kBK; kk += 16) {
        const bf16x8_t av = *reinterpret_cast<const bf16x8_t*>(xrow + k0 + kk + kgrp);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int col = b * 32 + (l & 31);
          uint16_t e[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) e[j] = stage[(kk + kgrp + j) * kStageStride + col];
          uint4 pk = make_uint4(e[0] | (uint32_t(e[1]) << 16), e[2] | (uint32_t(e[3]) << 16),
                                e[4] | (uint32_t(e[5]) << 16), e[6] | (uint32_t(e[7]) << 16));
          const bf16x8_t bv = __builtin_bit_cast(bf16x8_t, pk);
          acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc[b], 0, 0, 0);
        }
      }
    }
  }
  __syncthreads();
  // Partial tiles -> LDS red[w][32][128] (MFMA 32x32 output layout: lane l holds
  // column l % 32, rows 8 (i / 4) + 4 (l / 32) + i % 4).
  float* red = reinterpret_cast<float*>(region);
#pragma unroll
  for (int b = 0; b < 4; ++b) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = 8 * (i >> 2) + 4 * (l >> 5) + (i & 3);
      red[(w * kBM + r) * kCC + b * 32 + (l & 31)] = acc[b][i];
    }
  }
  __syncthreads();
  for (int o = tid; o < kBM * kCC; o += kThreads) {
    const int r = o / kCC, c = o % kCC;
    if (c0 + c >= a.E) continue;
    float v = red[(0 * kBM + r) * kCC + c];
    v += red[(1 * kBM + r) * kCC + c];
    v += red[(2 * kBM + r) * kCC + c];
    v += red[(3 * kBM + r) * kCC + c];
    lg[r * lgs + c0 + c] = v;
  }
  __syncthreads();
}

// float32 router: each thread forms whole dot products in order over c.
__device__ void router_f32(const RouteArgs& a, int t0, float* lg, int lgs) {
  const float* x = static_cast<const float*>(a.x);
  const float* wr = static_cast<const float*>(a.w_router);
  for (int o = threadIdx.x; o < kBM * a.E; o += kThreads) {
    const int r = o / a.E, e = o % a.E;
    const int t = min(t0 + r, a.T - 1);
    const float* xr = x + (size_t)t * a.d;
    float acc = 0.f;
    for (int c = 0; c < a.d; ++c) acc = fmaf(xr[c], wr[(size_t)c * a.E + e], acc);
    lg[r * lgs + e] = acc;
  }
  __syncthreads();
}

template <bool kBF16>
__global__ __launch_bounds__(kThreads) void route_kernel(RouteArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* region = smem;
  float* lg = reinterpret_cast<float*>(smem + kRegionBytes);
  const int lgs = a.E;  // row stride of the logit tile
  const int t0 = blockIdx.x * kBM;
  const int tid = threadIdx.x;

  if (a.w_router == nullptr) {
    for (int o = tid; o < kBM * a.E; o += kThreads) {
      const int r = o / a.E, e = o % a.E;
      const int t = min(t0 + r, a.T - 1);
      lg[r * lgs + e] = a.logits_in[(size_t)t * a.E + e];
    }
    __syncthreads();
  } else {
    if constexpr (kBF16) {
      for (int c0 = 0; c0 < a.E; c0 += kCC) router_pass_bf16(a, t0, c0, region, lg, lgs);
    } else {
      router_f32(a, t0, lg, lgs);
    }
    // bias, then publish the exact float32 values the selection will use
    for (int o = tid; o < kBM * a.E; o += kThreads) {
      const int r = o / a.E, e = o % a.E;
      float v = lg[r * lgs + e];
      if (a.bias) v += a.bias[e];
      lg[r * lgs + e] = v;
      if (a.logits_out && t0 + r < a.T) a.logits_out[(size_t)(t0 + r) * a.E + e] = v;
    }
    __syncthreads();
  }

  // Top-k and gates: wave w handles rows 8w .. 8w+7.
  const int w = tid / kWave;
  const int l = lane_id();
  const int per_lane = (a.E + kWave - 1) / kWave;  // <= 8 for E <= 512
  for (int rr = 0; rr < kBM / 4; ++rr) {
    const int r = w * (kBM / 4) + rr;
    const int t = t0 + r;
    if (t >= a.T) break;
    const float* row = lg + r * lgs;
    uint32_t taken = 0;  // bit j: expert l + 64 j already chosen
    float first = 0.f;
    float mine[8];       // chosen logit i is held by lane i % 64 in slot i / 64
#pragma unroll
    for (int q = 0; q < 8; ++q) mine[q] = 0.f;
    for (int i = 0; i < a.k; ++i) {
      float bv = -INFINITY;
      int be = 0x7fffffff;
      for (int j = 0; j < per_lane; ++j) {
        const int e = l + kWave * j;
        if (e >= a.E || ((taken >> j) & 1u)) continue;
        float v = row[e];
        if (v != v) v = -INFINITY;  // NaN never wins (inputs are expected finite)
        if (v > bv || (v == bv && e < be)) { bv = v; be = e; }
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        const float ov = __shfl_xor(bv, o, kWave);
        const int oe = __shfl_xor(be, o, kWave);
        if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
      }
      if ((be & (kWave - 1)) == l) taken |= 1u << (be / kWave);
      if (i == 0) first = bv;
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (i == q * kWave + l) mine[q] = bv;
      if (l == 0) a.topk_idx[(size_t)t * a.k + i] = be;
    }
    // gates: exp(L_i - L_0) / sum over the chosen, summed in a fixed tree order
    float part = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      if (q * kWave + l < a.k) {
        mine[q] = expf(mine[q] - first);
        part += mine[q];
      }
    }
    const float tot = wave_sum(part);
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (q * kWave + l < a.k) a.topk_w[(size_t)t * a.k + q * kWave + l] = mine[q] / tot;
  }
}

}  // namespace

hipError_t route(const Shape& s, const void* x, const void* w_router, const float* bias,
                 const float* logits_in, float* logits_out, int32_t* topk_idx, float* topk_w,
                 hipStream_t st) {
  if (s.T == 0) return hipSuccess;
  RouteArgs a{x, w_router, bias, logits_in, logits_out, topk_idx, topk_w, s.T, s.d, s.E, s.k};
  const size_t lds = kRegionBytes + (size_t)kBM * s.E * sizeof(float);
  const dim3 grid((s.T + kBM - 1) / kBM);
  static bool attr_set[2] = {false, false};
  const int which = s.act == kBF16 ? 1 : 0;
  const void* kern = which ? reinterpret_cast<const void*>(route_kernel<true>)
                           : reinterpret_cast<const void*>(route_kernel<false>);
  if (!attr_set[which]) {
    const int max_lds = kRegionBytes + kBM * kMaxExperts * (int)sizeof(float);
    hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, max_lds);
    if (e != hipSuccess) return e;
    attr_set[which] = true;
  }
  if (which) {
    hipLaunchKernelGGL(route_kernel<true>, grid, dim3(kThreads), lds, st, a);
  } else {
    hipLaunchKernelGGL(route_kernel<false>, grid, dim3(kThreads), lds, st, a);
  }
  return hipGetLastError();
}

}  // namespace moe
