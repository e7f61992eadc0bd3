// Router logits and softmax top-k gating on gfx950.
//
// "Wide Expert Parallelism" (llm-d notes), section "What is an MoE layer?":
// a small gate inspects every token and sends it to a few of the experts.
// Here: L = x W_r + b with float32 accumulation, the k largest L per token
// ordered by (-L, e) (ties to the lower expert index), and gates equal to a
// softmax over the k chosen logits (a softmax over all E renormalised over
// the chosen k: the full denominator cancels).
//
// Kernels:
//  * router_partial (bf16): workgroup (32-token tile, K split) forms the
//    32 x E partial products over its K range on MFMA 32x32x16; its four
//    waves take interleaved K steps and their partials are added in a fixed
//    order.  Splitting K gives a decode batch (T = 64) enough workgroups to
//    cover the chip.  Two variants: "staged" reads W_r as stored ([d][E],
//    coalesced along E) and transposes it through per-wave LDS buffers;
//    "direct" (up to 32 experts, one 32-wide MFMA block) reads a transposed
//    copy straight from global memory with a three-step prefetch.  float32:
//    plain FMAs;
//  * with many tokens and more than 128 experts, the expert GEMMs' pipeline
//    in router mode on the transposed copy (one split);
//  * router_transpose: W_r -> [E][d] in scratch, for the last two;
//  * router_topk: one wave per token adds the K-split partials in a fixed
//    order plus the bias, publishes the float32 logits, and selects the top k
//    on exactly those values; gates are exp(L_i - L_0) normalised over the k.
// Every sum has a fixed order, so the logits (and hence the routing) are
// bit-reproducible from run to run.
#include <type_traits>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kBM = 32;        // tokens per partial workgroup
constexpr int kThreads = 256;  // 4 waves
constexpr int kWaves = kThreads / kWave;

struct PartialArgs {
  const void* x;         // [T][d]
  const void* w;         // the router matrix: [d][E] (stored), or [E][d] (direct kernel)
  float* out;            // [nsplit][T][E] partial sums
  int T, d, E;
  int k_per_split;       // multiple of 128
};

// bf16 partial products, router matrix read in its stored [d][E] layout:
// workgroup (32-token tile, K split), four waves taking interleaved 32-deep K
// steps, each wave staging its own W_r rows (coalesced 16-byte loads along E)
// through a private LDS buffer and reading them back transposed for the MFMA,
// with the next step's loads in flight; 128 experts per pass; fixed-order sum
// of the four wave partials.  Used for more than 32 experts.
constexpr int kCC = 128;       // expert columns per pass (4 MFMA blocks of 32)
constexpr int kBK = 32;        // K rows of W_r per wave step
constexpr int kStageStride = kCC + 8;  // bf16 per staged W_r row (padded)
constexpr int kStageElems = kBK * kStageStride;


// Global loads of one 32-deep K step: W_r rows k0 + (l / 16) + 4 i, columns
// c0 + 8 (l % 16) .. +8, and this lane's two A fragments.
#define MOE_ROUTER_LOAD(STEP)                                                                 \
  do {                                                                                        \
    const int k0_ = kbeg + (STEP) * kBK;                                                      \
    if (full) {                                                                               \
      _Pragma("unroll") for (int i = 0; i < 8; ++i) rw[i] =                                   \
          *reinterpret_cast<const u32x4_t*>(wr + (size_t)(k0_ + sr + 4 * i) * a.E + c0 + sc); \
    } else {                                                                                  \
      _Pragma("unroll") for (int i = 0; i < 8; ++i) {                                         \
        uint32_t h_[4];                                                                       \
        _Pragma("unroll") for (int j = 0; j < 4; ++j) {                                       \
          const int col_ = c0 + sc + 2 * j;                                                   \
          const uint16_t* src_ = wr + (size_t)(k0_ + sr + 4 * i) * a.E + col_;                \
          const uint32_t lo_ = col_ < a.E ? src_[0] : 0u;                                     \
          const uint32_t hi_ = col_ + 1 < a.E ? src_[1] : 0u;                                 \
          h_[j] = lo_ | (hi_ << 16);                                                          \
        }                                                                                     \
        rw[i] = u32x4_t{h_[0], h_[1], h_[2], h_[3]};                                          \
      }                                                                                       \
    }                                                                                         \
    ra0 = *reinterpret_cast<const bf16x8_t*>(xrow + k0_ + kgrp);                              \
    ra1 = *reinterpret_cast<const bf16x8_t*>(xrow + k0_ + 16 + kgrp);                         \
  } while (0)

// LDS: the four wave stages during the K loop, then the four wave partials.
constexpr int kRouterLds = 4 * kBM * kCC * 4;  // 64 KB
static_assert(4 * kStageElems * 2 <= kRouterLds, "stages fit the shared region");

__global__ __launch_bounds__(kThreads) void router_partial_staged(PartialArgs a) {
  __shared__ __align__(16) unsigned char smem[kRouterLds];
  uint16_t (*stage)[kStageElems] = reinterpret_cast<uint16_t (*)[kStageElems]>(smem);
  float (*red)[kBM][kCC] = reinterpret_cast<float (*)[kBM][kCC]>(smem);
  const int tid = threadIdx.x;
  const int w = tid / kWave;
  const int l = lane_id();
  const int t0 = blockIdx.x * kBM;
  const int split = blockIdx.y;
  const int kbeg = split * a.k_per_split;
  const int nsteps = a.k_per_split / kBK;  // multiple of 4
  const uint16_t* x = static_cast<const uint16_t*>(a.x);
  const uint16_t* wr = static_cast<const uint16_t*>(a.w);
  uint16_t* st = stage[w];
  float* out = a.out + (size_t)split * a.T * a.E;

  // A rows: lane l serves token row l % 32 (clamped), 8 K values at 8 (l / 32).
  const int arow = min(t0 + (l & 31), a.T - 1);
  const uint16_t* xrow = x + (size_t)arow * a.d;
  const int kgrp = (l >> 5) * 8;
  const int sr = l >> 4, sc = (l & 15) * 8;

  for (int c0 = 0; c0 < a.E; c0 += kCC) {
    const bool full = (a.E & 7) == 0 && c0 + kCC <= a.E;  // wave-uniform
    f32x16_t acc[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[b] = f32x16_t{};
    u32x4_t rw[8];
    bf16x8_t ra0, ra1;

    int step = w;
    if (step < nsteps) MOE_ROUTER_LOAD(step);
    for (; step < nsteps; step += 4) {
      // registers -> this wave's private LDS stage.  LDS executes one wave's
      // operations in order, so the previous step's reads of the stage are
      // done before these writes land, and these writes before the reads
      // below; the empty asm only keeps the compiler from moving LDS accesses
      // across.
#pragma unroll
      for (int i = 0; i < 8; ++i)
        *reinterpret_cast<u32x4_t*>(st + (sr + 4 * i) * kStageStride + sc) = rw[i];
      const bf16x8_t a0 = ra0, a1 = ra1;
      asm volatile("" ::: "memory");
      if (step + 4 < nsteps) MOE_ROUTER_LOAD(step + 4);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const bf16x8_t av = h ? a1 : a0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int col = b * 32 + (l & 31);
          uint16_t e[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) e[j] = st[(h * 16 + kgrp + j) * kStageStride + col];
          const u32x4_t pk = {e[0] | (uint32_t(e[1]) << 16), e[2] | (uint32_t(e[3]) << 16),
                              e[4] | (uint32_t(e[5]) << 16), e[6] | (uint32_t(e[7]) << 16)};
          acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, __builtin_bit_cast(bf16x8_t, pk),
                                                           acc[b], 0, 0, 0);
        }
      }
      asm volatile("" ::: "memory");
    }
    // wave partials -> LDS (MFMA 32x32 layout: lane l holds column l % 32,
    // rows 8 (i / 4) + 4 (l / 32) + i % 4), then a fixed-order sum
    __syncthreads();  // every wave is done with its stage (same LDS)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        red[w][8 * (i >> 2) + 4 * (l >> 5) + (i & 3)][b * 32 + (l & 31)] = acc[b][i];
    __syncthreads();
    for (int o = tid; o < kBM * kCC; o += kThreads) {
      const int r = o / kCC, c = o % kCC;
      if (t0 + r < a.T && c0 + c < a.E)
        out[(size_t)(t0 + r) * a.E + c0 + c] =
            ((red[0][r][c] + red[1][r][c]) + red[2][r][c]) + red[3][r][c];
    }
    __syncthreads();
  }
}
#undef MOE_ROUTER_LOAD


// bf16 partial products on MFMA 32x32x16, straight from global memory (the
// router matrix transposed to [E][d] stays in L2; x rows stream once):
// workgroup (32-token tile, K split), four waves taking interleaved 16-deep K
// steps with loads three steps ahead, NB blocks of 32 experts per pass, and a
// fixed-order sum of the four wave partials through LDS.  Used for up to 32
// experts, where one 32-wide block covers them all.
template <int NB>
__global__ __launch_bounds__(kThreads) void router_partial_direct(PartialArgs a) {
  __shared__ float red[kWaves][kBM][NB * 32];
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int l = lane_id();
  const int t0 = blockIdx.x * kBM;
  const int split = blockIdx.y;
  const int kbeg = split * a.k_per_split;
  const int nsteps = a.k_per_split / 16;
  const uint16_t* x = static_cast<const uint16_t*>(a.x);
  const uint16_t* wt = static_cast<const uint16_t*>(a.w);
  float* out = a.out + (size_t)split * a.T * a.E;
  // lane l: token row l % 32 of the tile (A) / expert l % 32 of a block (B),
  // K values 8 (l / 32) .. + 8 of each 16-deep step
  const uint16_t* xrow = x + (size_t)min(t0 + (l & 31), a.T - 1) * a.d + kbeg + 8 * (l >> 5);
  for (int c0 = 0; c0 < a.E; c0 += NB * 32) {
    const uint16_t* wrow[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b)
      wrow[b] = wt + (size_t)min(c0 + b * 32 + (l & 31), a.E - 1) * a.d + kbeg + 8 * (l >> 5);
    f32x16_t acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] = f32x16_t{};
    // this wave's steps are s = w, w + 4, ...; loads run three steps ahead of
    // the MFMAs (four register sets).  Steps past the end contribute zero (A
    // set to 0), so every wave runs whole groups of four steps.
    bf16x8_t fa[4], fb[4][NB];
    bool live[4];
    auto load = [&](int s, int buf) {  // no branches: past the end, re-read the last step
      const int sc = min(s, nsteps - 1);
      live[buf] = s < nsteps;
      fa[buf] = *reinterpret_cast<const bf16x8_t*>(xrow + 16 * sc);
#pragma unroll
      for (int b = 0; b < NB; ++b)
        fb[buf][b] = *reinterpret_cast<const bf16x8_t*>(wrow[b] + 16 * sc);
    };
    auto mfma = [&](int buf) {
      // (the zero for a step past the end is chosen here, where the loads
      // are waited for anyway)
      const bf16x8_t av = live[buf] ? fa[buf] : bf16x8_t{};
#pragma unroll
      for (int b = 0; b < NB; ++b)  // tokens as the A operand: blocks are [token][expert]
        acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, fb[buf][b], acc[b], 0, 0, 0);
    };
    load(w, 0);
    load(w + kWaves, 1);
    load(w + 2 * kWaves, 2);
    // (scheduling barriers keep the compiler from pulling loads down to their
    // MFMAs, which would shorten the prefetch distance to nothing)
    for (int s = w; s < nsteps; s += 4 * kWaves) {
      load(s + 3 * kWaves, 3);
      __builtin_amdgcn_sched_barrier(0);
      mfma(0);
      __builtin_amdgcn_sched_barrier(0);
      load(s + 4 * kWaves, 0);
      __builtin_amdgcn_sched_barrier(0);
      mfma(1);
      __builtin_amdgcn_sched_barrier(0);
      load(s + 5 * kWaves, 1);
      __builtin_amdgcn_sched_barrier(0);
      mfma(2);
      __builtin_amdgcn_sched_barrier(0);
      load(s + 6 * kWaves, 2);
      __builtin_amdgcn_sched_barrier(0);
      mfma(3);
      __builtin_amdgcn_sched_barrier(0);
    }
    // wave partials -> LDS (lane l holds expert column l % 32 of each block,
    // token rows 8 (q / 4) + 4 (l / 32) + q % 4), then the fixed-order sum
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int q = 0; q < 16; ++q)
        red[w][8 * (q >> 2) + 4 * (l >> 5) + (q & 3)][b * 32 + (l & 31)] = acc[b][q];
    __syncthreads();
    for (int o = tid; o < kBM * NB * 32; o += kThreads) {
      const int r = o / (NB * 32), c = o % (NB * 32);
      if (t0 + r < a.T && c0 + c < a.E)
        out[(size_t)(t0 + r) * a.E + c0 + c] =
            ((red[0][r][c] + red[1][r][c]) + red[2][r][c]) + red[3][r][c];
    }
    __syncthreads();
  }
}

// float32 router on the fp32 matrix cores: workgroup (32-token tile, K
// split), 128 experts per pass, each wave one 32 x 32 block of
// v_mfma_f32_32x32x2_f32 (float32 products and sums).  Per 32-deep K stage
// the x tile and the router rows (read as stored, [d][E], consecutive lanes
// on consecutive experts) go to LDS K-major; the loads of the next two
// stages wait in registers and the LDS stages alternate between two
// buffers, one barrier per stage (the float32 problems are small, so a
// stage costs the latency of its loads).
constexpr int kRK = 32;  // K per stage
__global__ __launch_bounds__(kThreads) void router_partial_f32(PartialArgs a) {
  __shared__ float As[2][kRK][kBM];
  __shared__ float Bs[2][kRK][kCC];
  const float* x = static_cast<const float*>(a.x);
  const float* wr = static_cast<const float*>(a.w);
  const int tid = threadIdx.x;
  const int w = tid / kWave;
  const int l = lane_id();
  const int t0 = blockIdx.x * kBM;
  const int kbeg = blockIdx.y * a.k_per_split;
  const int nK = a.k_per_split / kRK;
  float* out = a.out + (size_t)blockIdx.y * a.T * a.E;
  // x: thread tid stages float4 (tid % 8) of token row tid / 8 (clamped);
  // W_r: rows tid / 32 + 8 i, experts c0 + tid % 32 + 32 q (0 past E)
  const int sr = tid / 8, sk = (tid % 8) * 4;
  const float* xsrc = x + (size_t)min(t0 + sr, a.T - 1) * a.d + kbeg + sk;
  const int wk = tid / 32, we = tid % 32;
  f32x4_t ra[2];
  float rb[2][4][4];
  for (int c0 = 0; c0 < a.E; c0 += kCC) {
    auto load = [&](int s, auto bc) {
      constexpr int b = decltype(bc)::value;
      ra[b] = *reinterpret_cast<const f32x4_t*>(xsrc + s * kRK);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float* row = wr + (size_t)(kbeg + s * kRK + wk + 8 * i) * a.E;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int e = c0 + we + 32 * q;
          rb[b][i][q] = e < a.E ? row[e] : 0.0f;
        }
      }
    };
    f32x16_t acc = f32x16_t{};
    auto stage = [&](int s, auto bc) {
      constexpr int b = decltype(bc)::value;
#pragma unroll
      for (int q = 0; q < 4; ++q) As[b][sk + q][sr] = ra[b][q];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) Bs[b][wk + 8 * i][we + 32 * q] = rb[b][i][q];
      __syncthreads();
      if (s + 2 < nK) load(s + 2, bc);
      // lane l gives A[token l % 32][k l / 32] and B[k l / 32][expert l % 32]
#pragma unroll
      for (int kk = 0; kk < kRK; kk += 2)
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(As[b][kk + l / 32][l % 32],
                                                   Bs[b][kk + l / 32][w * 32 + l % 32], acc, 0,
                                                   0, 0);
    };
    constexpr std::integral_constant<int, 0> kB0{};
    constexpr std::integral_constant<int, 1> kB1{};
    load(0, kB0);
    if (nK > 1) load(1, kB1);
    for (int s = 0; s < nK; s += 2) {
      stage(s, kB0);
      if (s + 1 < nK) stage(s + 1, kB1);
    }
    // lane l holds expert c0 + 32 w + l % 32, token rows 8 (r / 4) + 4 (l / 32) + r % 4
    const int e = c0 + w * 32 + l % 32;
    if (e < a.E) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = t0 + 8 * (r / 4) + 4 * (l / 32) + (r % 4);
        if (t < a.T) out[(size_t)t * a.E + e] = acc[r];
      }
    }
    __syncthreads();  // the next pass's first stage reuses LDS buffer 0
  }
}

// Wave-wide maximum of a 64-bit key, on VALU lane exchanges only (DPP inside
// rows of 16 lanes, then the gfx950 row-pair and half-wave swaps): every lane
// ends with the maximum.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t key) {
  auto dpp_step = [&](auto ctrl_tag) {
    constexpr int kCtrl = decltype(ctrl_tag)::value;
    const uint32_t lo = (uint32_t)key, hi = (uint32_t)(key >> 32);
    const uint32_t plo = __builtin_amdgcn_update_dpp(0u, lo, kCtrl, 0xF, 0xF, false);
    const uint32_t phi = __builtin_amdgcn_update_dpp(0u, hi, kCtrl, 0xF, 0xF, false);
    const uint64_t p = ((uint64_t)phi << 32) | plo;
    key = p > key ? p : key;
  };
  dpp_step(std::integral_constant<int, 0xB1>{});   // quad_perm [1,0,3,2]: lane ^ 1
  dpp_step(std::integral_constant<int, 0x4E>{});   // quad_perm [2,3,0,1]: lane ^ 2
  dpp_step(std::integral_constant<int, 0x141>{});  // row_half_mirror: the other quad of 8
  dpp_step(std::integral_constant<int, 0x140>{});  // row_mirror: the other half of 16
  // The swaps exchange a register between row pairs (16) and wave halves
  // (32); each lane then holds its own value and its partner's, in some
  // order, in the two results, for the high and low words alike.
  {
    const uint32_t lo = (uint32_t)key, hi = (uint32_t)(key >> 32);
    const auto l2 = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
    const auto h2 = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
    const uint64_t a = ((uint64_t)h2[0] << 32) | l2[0], b = ((uint64_t)h2[1] << 32) | l2[1];
    key = a > b ? a : b;
  }
  {
    const uint32_t lo = (uint32_t)key, hi = (uint32_t)(key >> 32);
    const auto l2 = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
    const auto h2 = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
    const uint64_t a = ((uint64_t)h2[0] << 32) | l2[0], b = ((uint64_t)h2[1] << 32) | l2[1];
    key = a > b ? a : b;
  }
  return key;
}

// Selection key of (logit v, expert e): larger key = larger v, then smaller
// e.  The float bits are mapped to an order-preserving unsigned integer
// (after -0 -> +0, so that the two zeros tie as equal values do).
__device__ __forceinline__ uint64_t select_key(float v, int e) {
  const uint32_t b = __float_as_uint(v + 0.0f);
  const uint32_t ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((uint64_t)ord << 32) | (uint32_t)~e;
}
__device__ __forceinline__ float key_value(uint64_t key) {
  const uint32_t ord = (uint32_t)(key >> 32);
  return __uint_as_float((ord & 0x80000000u) ? (ord & 0x7fffffffu) : ~ord);
}

// One wave per token: logits = sum of the split partials (in split order) +
// bias; then top-k by (-L, e) and the renormalised gates.  Lane l holds
// experts l + 64 j (j < kPerLane).
template <int kPerLane>
__global__ __launch_bounds__(kThreads) void router_topk_kernel(const float* part, int nsplit,
                                                               const float* bias,
                                                               float* logits_out, int T, int E,
                                                               int k, int32_t* topk_idx,
                                                               float* topk_w) {
  const int w = threadIdx.x / kWave;
  const int l = lane_id();
  const int t = blockIdx.x * (kThreads / kWave) + w;
  if (t >= T) return;
  // split partials loaded together: all 16 splits of a decode batch in one
  // round of loads when E <= 128
  constexpr int kBatch = kPerLane <= 2 ? 16 : 8;
  float v[kPerLane];
#pragma unroll
  for (int j = 0; j < kPerLane; ++j) v[j] = 0.f;
  // sum over the splits in split order; each batch's loads are issued together
  for (int q0 = 0; q0 < nsplit; q0 += kBatch) {
    float pv[kPerLane][kBatch];
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) {
      const int e = l + kWave * j;
#pragma unroll
      for (int b = 0; b < kBatch; ++b)
        pv[j][b] = (e < E && q0 + b < nsplit) ? part[((size_t)(q0 + b) * T + t) * E + e] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) {
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        if (q0 + b < nsplit) v[j] = (q0 + b == 0) ? pv[j][b] : v[j] + pv[j][b];
      }
    }
  }
  uint64_t key[kPerLane];
#pragma unroll
  for (int j = 0; j < kPerLane; ++j) {
    const int e = l + kWave * j;
    key[j] = 0;  // below every real key: never chosen
    if (e < E) {
      float s = v[j];
      if (bias) s += bias[e];
      if (logits_out) logits_out[(size_t)t * E + e] = s;
      if (s != s) s = -INFINITY;  // NaN never wins (inputs are expected finite)
      key[j] = select_key(s, e);
    }
  }
  float first = 0.f;
  float mine[kMaxExperts / kWave];  // chosen logit i is held by lane i % 64 in slot i / 64
#pragma unroll
  for (int q = 0; q < kMaxExperts / kWave; ++q) mine[q] = 0.f;
  for (int i = 0; i < k; ++i) {
    uint64_t best = 0;
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) best = key[j] > best ? key[j] : best;
    best = wave_max_u64(best);
    const int be = (int)~(uint32_t)best;
    const float bv = key_value(best);
    if ((be & (kWave - 1)) == l) {  // the owner retires the chosen expert
#pragma unroll
      for (int j = 0; j < kPerLane; ++j)
        if (j == be / kWave) key[j] = 0;
    }
    if (i == 0) first = bv;
#pragma unroll
    for (int q = 0; q < kMaxExperts / kWave; ++q)
      if (i == q * kWave + l) mine[q] = bv;
    if (l == 0) topk_idx[(size_t)t * k + i] = be;
  }
  float psum = 0.f;
#pragma unroll
  for (int q = 0; q < kMaxExperts / kWave; ++q) {
    if (q * kWave + l < k) {
      mine[q] = expf(mine[q] - first);
      psum += mine[q];
    }
  }
  const float tot = wave_sum(psum);
#pragma unroll
  for (int q = 0; q < kMaxExperts / kWave; ++q)
    if (q * kWave + l < k) topk_w[(size_t)t * k + q * kWave + l] = mine[q] / tot;
}

// Maximum of a 64-bit key over each row of 16 lanes (DPP steps only): every
// lane of the row ends with the row's maximum.
__device__ __forceinline__ uint64_t row_max_u64(uint64_t key) {
  auto dpp_step = [&](auto ctrl_tag) {
    constexpr int kCtrl = decltype(ctrl_tag)::value;
    const uint32_t lo = (uint32_t)key, hi = (uint32_t)(key >> 32);
    const uint32_t plo = __builtin_amdgcn_update_dpp(0u, lo, kCtrl, 0xF, 0xF, false);
    const uint32_t phi = __builtin_amdgcn_update_dpp(0u, hi, kCtrl, 0xF, 0xF, false);
    const uint64_t p = ((uint64_t)phi << 32) | plo;
    key = p > key ? p : key;
  };
  dpp_step(std::integral_constant<int, 0xB1>{});   // quad_perm [1,0,3,2]: lane ^ 1
  dpp_step(std::integral_constant<int, 0x4E>{});   // quad_perm [2,3,0,1]: lane ^ 2
  dpp_step(std::integral_constant<int, 0x141>{});  // row_half_mirror: the other quad of 8
  dpp_step(std::integral_constant<int, 0x140>{});  // row_mirror: the other half of 16
  return key;
}

// Many tokens: a row of 16 lanes per token (four tokens per wave), lane j of
// the row holding experts j + 16 i (i < kPerLane), so that a selection round
// is a local maximum over kPerLane keys and four DPP steps instead of a
// wave-wide reduction per token.  Same sums, keys, ties and gates as
// router_topk_kernel; k <= 16 (chosen i is kept by lane i of the row).
template <int kPerLane>
__global__ __launch_bounds__(kThreads) void router_topk_rows_kernel(
    const float* part, int nsplit, const float* bias, float* logits_out, int T, int E, int k,
    int32_t* topk_idx, float* topk_w) {
  const int l = lane_id();
  const int j = l & 15;  // lane in the token's row
  const int t = (blockIdx.x * kThreads + threadIdx.x) / 16;
  const bool live = t < T;  // every lane takes part in the row exchanges
  float v[kPerLane];
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) v[i] = 0.f;
  for (int q = 0; q < nsplit; ++q) {
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
      const int e = j + 16 * i;
      const float pv = (live && e < E) ? part[((size_t)q * T + t) * E + e] : 0.f;
      v[i] = q == 0 ? pv : v[i] + pv;
    }
  }
  uint64_t key[kPerLane];
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) {
    const int e = j + 16 * i;
    key[i] = 0;  // below every real key: never chosen
    if (live && e < E) {
      float s = v[i];
      if (bias) s += bias[e];
      if (logits_out) logits_out[(size_t)t * E + e] = s;
      if (s != s) s = -INFINITY;  // NaN never wins (inputs are expected finite)
      key[i] = select_key(s, e);
    }
  }
  float first = 0.f, mine = 0.f;
  int mine_e = 0;
  for (int r = 0; r < k; ++r) {
    uint64_t best = key[0];
#pragma unroll
    for (int i = 1; i < kPerLane; ++i) best = key[i] > best ? key[i] : best;
    best = row_max_u64(best);
    // the owner retires the chosen expert (keys are distinct: they hold the id)
#pragma unroll
    for (int i = 0; i < kPerLane; ++i)
      if (key[i] == best) key[i] = 0;
    const float bv = key_value(best);
    if (r == 0) first = bv;
    if (r == j) {
      mine = bv;
      mine_e = (int)~(uint32_t)best;
    }
  }
  float p = j < k ? expf(mine - first) : 0.f;
  float tot = p;
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) tot += __shfl_xor(tot, o, kWave);
  if (live && j < k) {
    topk_idx[(size_t)t * k + j] = mine_e;
    topk_w[(size_t)t * k + j] = p / tot;
  }
}

// W_r [d][E] -> [E][d] (bf16), 64 x 64 tiles through LDS with 16-byte global
// accesses: the router kernels read each expert's weights as one contiguous
// K row, like the expert GEMMs.
__global__ __launch_bounds__(256) void router_transpose_bf16(const uint16_t* w, uint16_t* wt,
                                                             int d, int E) {
  __shared__ __align__(16) uint16_t tile[64][72];  // [k][e], 144-byte rows
  const int k0 = blockIdx.x * 64, e0 = blockIdx.y * 64;
  const bool full = (E % 8) == 0 && e0 + 64 <= E;
  for (int i = threadIdx.x; i < 512; i += 256) {
    const int r = i / 8, c = (i % 8) * 8;  // K row r, experts c .. c + 7
    const uint16_t* src = w + (size_t)(k0 + r) * E + e0 + c;
    if (full) {
      *reinterpret_cast<u32x4_t*>(&tile[r][c]) = *reinterpret_cast<const u32x4_t*>(src);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) tile[r][c + j] = e0 + c + j < E ? src[j] : uint16_t(0);
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 512; i += 256) {
    const int e = i / 8, c = (i % 8) * 8;  // expert e, K values c .. c + 7
    if (e0 + e < E) {
      u32x4_t v;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        v[j] = uint32_t(tile[c + 2 * j][e]) | (uint32_t(tile[c + 2 * j + 1][e]) << 16);
      *reinterpret_cast<u32x4_t*>(wt + (size_t)(e0 + e) * d + k0 + c) = v;
    }
  }
}

}  // namespace

int router_splits(const Shape& s) {
  // K splits for about one workgroup per compute unit, each split >= 128 deep
  const int tiles = (s.T + kBM - 1) / kBM;
  int splits = 1;
  while (s.d % (splits * 2 * 128) == 0 && tiles * splits * 2 <= 256) splits *= 2;
  return splits;
}

namespace {
// Router plans (bf16): up to 32 experts, the direct kernel on the transposed
// matrix; many tokens and more than 128 experts, the GEMM pipeline on the
// transposed matrix; otherwise the staged kernel on the stored matrix.
bool gemm_router(const Shape& s) { return use_router_gemm(s) && s.E > 128; }
bool direct_router(const Shape& s) { return s.act == kBF16 && s.E <= 32; }
// scratch layout: the transposed router matrix [E][d] bf16 (direct and GEMM
// plans), then the K-split partial sums [splits][T][E] float32 (more than one
// split)
size_t wt_bytes(const Shape& s) {
  return (gemm_router(s) || direct_router(s)) ? align_up((size_t)s.E * s.d * 2) : 0;
}
int splits_of(const Shape& s) { return gemm_router(s) ? router_gemm_splits(s) : router_splits(s); }
}  // namespace

size_t route_ws_bytes(const Shape& s) {
  const int ns = splits_of(s);
  return wt_bytes(s) + (ns > 1 ? align_up((size_t)ns * s.T * s.E * sizeof(float)) : 0);
}

hipError_t route(const Shape& s, const void* x, const void* w_router, const float* bias,
                 const float* logits_in, float* logits, int32_t* topk_idx, float* topk_w,
                 void* scratch, hipStream_t st) {
  if (s.T == 0) return hipSuccess;
  const float* part;
  const float* b = bias;
  int nsplit = 1;
  float* publish = logits;
  if (w_router == nullptr) {
    part = logits_in;  // final logits given: no bias, nothing to publish
    b = nullptr;
    publish = nullptr;
  } else {
    unsigned char* ws = static_cast<unsigned char*>(scratch);
    nsplit = splits_of(s);
    float* partials = nsplit > 1 ? reinterpret_cast<float*>(ws + wt_bytes(s)) : logits;
    hipError_t e = hipSuccess;
    const dim3 grid((s.T + kBM - 1) / kBM, nsplit);
    if (s.act == kBF16 && (gemm_router(s) || direct_router(s))) {
      // the router matrix as [E][d]: every expert's weights one contiguous K row
      uint16_t* wt = reinterpret_cast<uint16_t*>(ws);
      hipLaunchKernelGGL(router_transpose_bf16, dim3(s.d / 64, (s.E + 63) / 64), dim3(256), 0,
                         st, static_cast<const uint16_t*>(w_router), wt, s.d, s.E);
      e = hipGetLastError();
      if (e == hipSuccess && gemm_router(s)) {
        // many tokens and experts: x W_r from the expert GEMMs' pipeline
        e = router_gemm(s, x, wt, partials, st);
      } else if (e == hipSuccess) {
        PartialArgs pa{x, wt, partials, s.T, s.d, s.E, s.d / nsplit};
        hipLaunchKernelGGL(router_partial_direct<1>, grid, dim3(kThreads), 0, st, pa);
        e = hipGetLastError();
      }
    } else if (s.act == kBF16) {
      PartialArgs pa{x, w_router, partials, s.T, s.d, s.E, s.d / nsplit};
      hipLaunchKernelGGL(router_partial_staged, grid, dim3(kThreads), 0, st, pa);
      e = hipGetLastError();
    } else {
      PartialArgs pa{x, w_router, partials, s.T, s.d, s.E, s.d / nsplit};
      hipLaunchKernelGGL(router_partial_f32, grid, dim3(kThreads), 0, st, pa);
      e = hipGetLastError();
    }
    if (e != hipSuccess) return e;
    part = partials;
  }
  // (with one split the partials are `logits` itself: each lane reads its
  // elements, then writes the final values back)
  if (s.T >= 1024 && s.k <= 16) {
    // many tokens: four per wave
    const dim3 rgrid((s.T + kThreads / 16 - 1) / (kThreads / 16));
    if (s.E <= 64)
      hipLaunchKernelGGL(router_topk_rows_kernel<4>, rgrid, dim3(kThreads), 0, st, part, nsplit,
                         b, publish, s.T, s.E, s.k, topk_idx, topk_w);
    else if (s.E <= 128)
      hipLaunchKernelGGL(router_topk_rows_kernel<8>, rgrid, dim3(kThreads), 0, st, part, nsplit,
                         b, publish, s.T, s.E, s.k, topk_idx, topk_w);
    else if (s.E <= 256)
      hipLaunchKernelGGL(router_topk_rows_kernel<16>, rgrid, dim3(kThreads), 0, st, part, nsplit,
                         b, publish, s.T, s.E, s.k, topk_idx, topk_w);
    else
      hipLaunchKernelGGL(router_topk_rows_kernel<32>, rgrid, dim3(kThreads), 0, st, part, nsplit,
                         b, publish, s.T, s.E, s.k, topk_idx, topk_w);
    return hipGetLastError();
  }
  const int wpb = kThreads / kWave;
  const dim3 tgrid((s.T + wpb - 1) / wpb);
  if (s.E <= 64)
    hipLaunchKernelGGL(router_topk_kernel<1>, tgrid, dim3(kThreads), 0, st, part, nsplit, b,
                       publish, s.T, s.E, s.k, topk_idx, topk_w);
  else if (s.E <= 128)
    hipLaunchKernelGGL(router_topk_kernel<2>, tgrid, dim3(kThreads), 0, st, part, nsplit, b,
                       publish, s.T, s.E, s.k, topk_idx, topk_w);
  else if (s.E <= 256)
    hipLaunchKernelGGL(router_topk_kernel<4>, tgrid, dim3(kThreads), 0, st, part, nsplit, b,
                       publish, s.T, s.E, s.k, topk_idx, topk_w);
  else
    hipLaunchKernelGGL(router_topk_kernel<8>, tgrid, dim3(kThreads), 0, st, part, nsplit, b,
                       publish, s.T, s.E, s.k, topk_idx, topk_w);
  return hipGetLastError();
}

}  // namespace moe
