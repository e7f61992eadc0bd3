// Local experts: each expert's SwiGLU feed-forward network as a grouped GEMM
// over the ragged per-expert row segments of the dispatch order.
//
// "Serving MoE models with expert parallelism on 8xH200" (reviosa), section
// "Tensor parallel vs expert parallel": a GPU that owns whole experts runs
// full-size expert GEMMs on the tokens sent to it.  Section "Batching: MoE
// needs bigger batches than you think": at decode batch sizes each expert sees
// a handful of tokens and the expert GEMM only streams its weights from HBM;
// prefill gives each expert many rows.  Both regimes use the kernels below,
// with a 32-row tile for the first and a 128-row tile for the second.
//
//   gate/up:  h[p] = silu(A_p Wg_j) * (A_p Wu_j),  A_p = x[sorted_slot[p] / k]
//   down:     y[p] = (h[p] Wd_j) * gate(p)
//
// Structure (bf16 activations; bf16 or FP8-E4M3 weights):
//  * a one-workgroup schedule kernel splits every expert segment into M tiles
//    of BM rows and writes the (expert, first row) list and its length;
//  * a persistent GEMM kernel walks items (M tile, N tile); the items are cut
//    into eight contiguous ranges, one per XCD (workgroup b runs on XCD b % 8),
//    so items that share an A tile or a weight tile meet in the same L2;
//  * per item, a K loop of 64-deep steps: global -> registers (A rows gathered
//    through sorted_slot, weight rows streamed; FP8 codes widened exactly to
//    bf16) -> LDS (double buffered, 16-byte chunks XOR-swizzled by row) ->
//    MFMA 32x32x16 bf16 with float32 accumulation;
//  * FP8 weights carry a float32 scale per 128x128 block: the MFMA partial of
//    each 128-deep K block is accumulated separately and added to the running
//    sum times its block's scale, so the weights enter MFMA unrounded;
//  * epilogues: silu(gate) * up rounded to bf16 (gate/up), or the product
//    times the token's gate (down).
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kBK = 64;  // K elements per pipeline step
constexpr int kNumXcd = 8;

__global__ __launch_bounds__(kMaxExperts) void ffn_schedule_kernel(const int32_t* offsets, int El,
                                                                   int BM, int2* tiles,
                                                                   int* ntiles) {
  __shared__ int sums[kMaxExperts];
  const int e = threadIdx.x;
  const int lo = e < El ? offsets[e] : 0;
  const int cnt = e < El ? offsets[e + 1] - lo : 0;
  const int nt = (cnt + BM - 1) / BM;
  sums[e] = nt;
  __syncthreads();
  for (int o = 1; o < kMaxExperts; o <<= 1) {
    const int v = e >= o ? sums[e - o] : 0;
    __syncthreads();
    sums[e] += v;
    __syncthreads();
  }
  const int first = sums[e] - nt;
  for (int i = 0; i < nt; ++i) tiles[first + i] = make_int2(e, lo + i * BM);
  if (e == El - 1) *ntiles = sums[e];
}

struct GemmArgs {
  const uint16_t* A;           // gate/up: x [T][K]; down: h [S][K]  (bf16)
  const int32_t* sorted_slot;  // gate/up gather
  int k;                       // top-k (slot -> token)
  const void* W0;              // gate (gate/up) or down weights
  const void* W1;              // up weights (gate/up)
  const float* S0;             // FP8 scales for W0
  const float* S1;             // FP8 scales for W1
  const float* topk_w;         // down epilogue gates, or null
  uint16_t* out;               // gate/up: h [S][Nout]; down: y [S][Nout]
  const int32_t* offsets;      // [El + 1]
  const int2* tiles;           // (expert, row0)
  const int* ntiles;
  int K;                       // reduction length
  int Nout;                    // output columns
  int n_tiles_n;               // N tiles per M tile
};

// Byte offset of 16-byte chunk c (0..7) of row r in a [rows][64] bf16 LDS tile.
__device__ __forceinline__ int swz(int r, int c) { return r * 128 + ((c ^ (r & 7)) << 4); }

template <int MB, int WM, int NB, int WN, bool kGateUp, bool kFP8>
struct Cfg {
  static constexpr int kThreads = kWave * WM * WN;
  static constexpr int BM = 32 * MB * WM;    // tile rows
  static constexpr int BNW = 32 * NB * WN;   // weight rows per tile
  static constexpr int kAChunks = BM * 8 / kThreads;             // 16-byte A chunks / thread
  static constexpr int kBChunks = BNW * (kFP8 ? 4 : 8) / kThreads;  // 16-byte B chunks / thread
  static constexpr int kLdsA = BM * 128;     // bytes per A stage
  static constexpr int kLdsB = BNW * 128;    // bytes per B stage (bf16 after widening)
  static constexpr int kLds = 2 * (kLdsA + kLdsB);
  static_assert(BM * 8 % kThreads == 0 && BNW * (kFP8 ? 4 : 8) % kThreads == 0, "load split");
  static_assert(!kGateUp || NB % 2 == 0, "gate/up pairs column blocks");
};

template <int MB, int WM, int NB, int WN, bool kGateUp, bool kFP8, int kMinBlocks>
__global__ __launch_bounds__(kWave* WM* WN, kMinBlocks) void grouped_gemm_kernel(GemmArgs a) {
  using C = Cfg<MB, WM, NB, WN, kGateUp, kFP8>;
  constexpr int NT = C::kThreads;
  constexpr int BNW = C::BNW;
  extern __shared__ __align__(16) unsigned char smem[];
  // stage buffers: A0 A1 B0 B1
  auto ldsA = [&](int buf) { return smem + buf * C::kLdsA; };
  auto ldsB = [&](int buf) { return smem + 2 * C::kLdsA + buf * C::kLdsB; };

  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int l = lane_id();
  const int wm = wave % WM;
  const int wn = wave / WM;
  const int welem = kFP8 ? 1 : 2;  // bytes per weight element

  // persistent, XCD-contiguous item ranges
  const int n_items = *a.ntiles * a.n_tiles_n;
  const int xcd = blockIdx.x % kNumXcd;
  const int per_xcd = gridDim.x / kNumXcd;
  const int slot = blockIdx.x / kNumXcd;
  const int it_begin = (int)((long long)n_items * xcd / kNumXcd);
  const int it_end = (int)((long long)n_items * (xcd + 1) / kNumXcd);

  for (int item = it_begin + slot; item < it_end; item += per_xcd) {
    const int g = item / a.n_tiles_n;
    const int nt = item % a.n_tiles_n;
    const int2 tile = a.tiles[g];
    const int j = tile.x;
    const int row0 = tile.y;
    const int row_end = a.offsets[j + 1];
    // first output column (gate/up: h column; down: y column) of this tile
    const int n0 = nt * (kGateUp ? BNW / 2 : BNW);

    // ---- per-thread global source pointers for this tile
    const uint16_t* a_src[C::kAChunks];
#pragma unroll
    for (int i = 0; i < C::kAChunks; ++i) {
      const int q = tid + i * NT;
      const int r = q >> 3;
      const int p = min(row0 + r, row_end - 1);
      const long long arow = kGateUp ? (long long)(a.sorted_slot[p] / a.k) : (long long)p;
      a_src[i] = a.A + arow * a.K + (q & 7) * 8;
    }
    const unsigned char* b_src[C::kBChunks];
#pragma unroll
    for (int i = 0; i < C::kBChunks; ++i) {
      const int q = tid + i * NT;
      const int r = kFP8 ? (q >> 2) : (q >> 3);  // weight row in tile
      const int c = kFP8 ? (q & 3) : (q & 7);    // 16-byte chunk in the 64-deep step
      const unsigned char* base;
      int wrow;
      if (kGateUp) {
        const bool up = r >= BNW / 2;
        wrow = n0 + (up ? r - BNW / 2 : r);
        base = static_cast<const unsigned char*>(up ? a.W1 : a.W0);
      } else {
        wrow = min(n0 + r, a.Nout - 1);
        base = static_cast<const unsigned char*>(a.W0);
      }
      b_src[i] = base + ((long long)j * a.Nout + wrow) * a.K * welem + c * 16;
    }

    u32x4_t ra[C::kAChunks];
    u32x4_t rb[C::kBChunks];
// global -> registers for K step KS
#define MOE_GLOAD(KS)                                                                       \
  do {                                                                                      \
    _Pragma("unroll") for (int i = 0; i < C::kAChunks; ++i) ra[i] =                         \
        *reinterpret_cast<const u32x4_t*>(a_src[i] + (KS) * kBK);                           \
    _Pragma("unroll") for (int i = 0; i < C::kBChunks; ++i) rb[i] =                         \
        *reinterpret_cast<const u32x4_t*>(b_src[i] + (long long)(KS) * kBK * welem);          \
  } while (0)
// registers -> LDS stage BUF (FP8 codes widened to bf16 on the way)
#define MOE_LSTORE(BUF)                                                                     \
  do {                                                                                      \
    _Pragma("unroll") for (int i = 0; i < C::kAChunks; ++i) {                               \
      const int q = tid + i * NT;                                                           \
      *reinterpret_cast<u32x4_t*>(ldsA(BUF) + swz(q >> 3, q & 7)) = ra[i];                  \
    }                                                                                       \
    _Pragma("unroll") for (int i = 0; i < C::kBChunks; ++i) {                               \
      const int q = tid + i * NT;                                                           \
      if constexpr (kFP8) {                                                                 \
        const int r = q >> 2, c = q & 3;                                                    \
        const u32x2_t w0 = e4m3x4_to_bf16x4(rb[i].x), w1 = e4m3x4_to_bf16x4(rb[i].y);       \
        const u32x2_t w2 = e4m3x4_to_bf16x4(rb[i].z), w3 = e4m3x4_to_bf16x4(rb[i].w);       \
        *reinterpret_cast<u32x4_t*>(ldsB(BUF) + swz(r, 2 * c)) =                            \
            u32x4_t{w0.x, w0.y, w1.x, w1.y};                                                \
        *reinterpret_cast<u32x4_t*>(ldsB(BUF) + swz(r, 2 * c + 1)) =                        \
            u32x4_t{w2.x, w2.y, w3.x, w3.y};                                                \
      } else {                                                                              \
        *reinterpret_cast<u32x4_t*>(ldsB(BUF) + swz(q >> 3, q & 7)) = rb[i];                \
      }                                                                                     \
    }                                                                                       \
  } while (0)

    f32x16_t acc[MB][NB];
    f32x16_t part[kFP8 ? MB : 1][kFP8 ? NB : 1];
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int n = 0; n < NB; ++n) acc[m][n] = f32x16_t{};
    if constexpr (kFP8) {
#pragma unroll
      for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int n = 0; n < NB; ++n) part[m][n] = f32x16_t{};
    }

    // LDS row of MFMA block rows for this wave
    const int arow_base = wm * MB * 32 + (l & 31);
    auto brow = [&](int n) -> int {
      if (kGateUp) {
        constexpr int H = NB / 2;
        return (n < H ? 0 : BNW / 2) + wn * H * 32 + (n % H) * 32 + (l & 31);
      }
      return wn * NB * 32 + n * 32 + (l & 31);
    };

    const int nK = a.K / kBK;
    __syncthreads();  // LDS of the previous item is no longer read
    MOE_GLOAD(0);
    MOE_LSTORE(0);
    __syncthreads();
    for (int ks = 0; ks < nK; ++ks) {
      const int cur = ks & 1;
      if (ks + 1 < nK) MOE_GLOAD(ks + 1);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int c = kk * 2 + (l >> 5);
        bf16x8_t af[MB];
#pragma unroll
        for (int m = 0; m < MB; ++m)
          af[m] = *reinterpret_cast<const bf16x8_t*>(ldsA(cur) + swz(arow_base + m * 32, c));
#pragma unroll
        for (int n = 0; n < NB; ++n) {
          const bf16x8_t bfr = *reinterpret_cast<const bf16x8_t*>(ldsB(cur) + swz(brow(n), c));
#pragma unroll
          for (int m = 0; m < MB; ++m) {
            if constexpr (kFP8)
              part[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[m], bfr, part[m][n], 0, 0, 0);
            else
              acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[m], bfr, acc[m][n], 0, 0, 0);
          }
        }
      }
      if constexpr (kFP8) {
        if (ks & 1) {  // end of a 128-deep scale block
          const int kb = ks >> 1;
          const int kblocks = a.K / 128;
          float sc[NB];
#pragma unroll
          for (int n = 0; n < NB; ++n) {
            int nrow;  // first matrix row of the block -> its 128-row scale block
            const float* S;
            if (kGateUp) {
              constexpr int H = NB / 2;
              nrow = n0 + wn * H * 32 + (n % H) * 32;
              S = n < H ? a.S0 : a.S1;
            } else {
              nrow = min(n0 + wn * NB * 32 + n * 32, a.Nout - 1);
              S = a.S0;
            }
            sc[n] = S[((long long)j * (a.Nout / 128) + nrow / 128) * kblocks + kb];
          }
#pragma unroll
          for (int m = 0; m < MB; ++m)
#pragma unroll
            for (int n = 0; n < NB; ++n) {
              acc[m][n] += part[m][n] * sc[n];
              part[m][n] = f32x16_t{};
            }
        }
      }
      if (ks + 1 < nK) MOE_LSTORE(cur ^ 1);
      __syncthreads();
    }

    // ---- epilogue (MFMA 32x32 layout: lane l holds column l % 32 and rows
    // 8 (i / 4) + 4 (l / 32) + (i % 4) of each block)
#pragma unroll
    for (int m = 0; m < MB; ++m) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = wm * MB * 32 + m * 32 + 8 * (i >> 2) + 4 * (l >> 5) + (i & 3);
        const int p = row0 + r;
        if (p >= row_end) continue;
        if constexpr (kGateUp) {
          constexpr int H = NB / 2;
#pragma unroll
          for (int n = 0; n < H; ++n) {
            const int col = n0 + wn * H * 32 + n * 32 + (l & 31);
            const float gv = acc[m][n][i], uv = acc[m][n + H][i];
            a.out[(long long)p * a.Nout + col] = f32_to_bf16(silu_f32(gv) * uv);
          }
        } else {
          const float gw = a.topk_w ? a.topk_w[a.sorted_slot[p]] : 1.0f;
#pragma unroll
          for (int n = 0; n < NB; ++n) {
            const int col = n0 + wn * NB * 32 + n * 32 + (l & 31);
            if (col < a.Nout) a.out[(long long)p * a.Nout + col] = f32_to_bf16(acc[m][n][i] * gw);
          }
        }
      }
    }
  }
}

#undef MOE_GLOAD
#undef MOE_LSTORE

// ---- float32 path: plain VALU dot products over the same tile schedule
constexpr int kF32BM = 32;
constexpr int kF32BN = 64;

template <bool kGateUp>
__global__ __launch_bounds__(256) void grouped_f32_kernel(GemmArgs a) {
  const int n_items = *a.ntiles * a.n_tiles_n;
  const float* A = reinterpret_cast<const float*>(a.A);
  const float* W0 = static_cast<const float*>(a.W0);
  const float* W1 = static_cast<const float*>(a.W1);
  float* out = reinterpret_cast<float*>(a.out);
  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int g = item / a.n_tiles_n;
    const int nt = item % a.n_tiles_n;
    const int2 tile = a.tiles[g];
    const int j = tile.x, row0 = tile.y;
    const int row_end = a.offsets[j + 1];
    for (int o = threadIdx.x; o < kF32BM * kF32BN; o += blockDim.x) {
      const int r = o / kF32BN, c = o % kF32BN;
      const int p = row0 + r;
      const int col = nt * kF32BN + c;
      if (p >= row_end || col >= a.Nout) continue;
      const long long arow = kGateUp ? (long long)(a.sorted_slot[p] / a.k) : (long long)p;
      const float* ar = A + arow * a.K;
      const float* w0 = W0 + ((long long)j * a.Nout + col) * a.K;
      if (kGateUp) {
        const float* w1 = W1 + ((long long)j * a.Nout + col) * a.K;
        float gs = 0.f, us = 0.f;
        for (int q = 0; q < a.K; ++q) {
          gs = fmaf(ar[q], w0[q], gs);
          us = fmaf(ar[q], w1[q], us);
        }
        out[(long long)p * a.Nout + col] = gs / (1.0f + expf(-gs)) * us;
      } else {
        float ys = 0.f;
        for (int q = 0; q < a.K; ++q) ys = fmaf(ar[q], w0[q], ys);
        const float gw = a.topk_w ? a.topk_w[a.sorted_slot[p]] : 1.0f;
        out[(long long)p * a.Nout + col] = ys * gw;
      }
    }
  }
}

// ---- launch plumbing
int g_num_cu = 0;

int num_cu() {
  if (g_num_cu == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      g_num_cu = n;
    else
      g_num_cu = 256;
  }
  return g_num_cu;
}

template <int MB, int WM, int NB, int WN, bool kGateUp, bool kFP8, int kMinBlocks>
hipError_t launch_gemm(const GemmArgs& a, long long max_items, hipStream_t st) {
  using C = Cfg<MB, WM, NB, WN, kGateUp, kFP8>;
  auto kern = grouped_gemm_kernel<MB, WM, NB, WN, kGateUp, kFP8, kMinBlocks>;
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, C::kLds);
    if (e != hipSuccess) return e;
    attr = true;
  }
  long long grid = (long long)num_cu() * kMinBlocks;
  const long long need = (max_items + kNumXcd - 1) / kNumXcd * kNumXcd;
  if (need < grid) grid = need;
  grid = (grid + kNumXcd - 1) / kNumXcd * kNumXcd;
  if (grid < kNumXcd) grid = kNumXcd;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(C::kThreads), C::kLds, st, a);
  return hipGetLastError();
}

// Tile shapes: decode (few rows per expert) and prefill (many rows).
constexpr int kDecodeBM = 32;    // MB=1, WM=1
constexpr int kPrefillBM = 128;  // MB=2, WM=2

bool use_decode_tiles(const Shape& s) { return s.S <= 64LL * s.El; }

int tile_bm(const Shape& s) {
  if (s.weight == kF32) return kF32BM;
  return use_decode_tiles(s) ? kDecodeBM : kPrefillBM;
}

size_t max_tiles(const Shape& s, int bm) { return (size_t)((s.S + bm - 1) / bm) + s.El; }

}  // namespace

FfnSchedule ffn_schedule_view(const Shape& s, void* ws) {
  unsigned char* p = static_cast<unsigned char*>(ws);
  FfnSchedule v;
  v.tiles = reinterpret_cast<int2*>(p);
  v.ntiles = reinterpret_cast<int*>(p + align_up(max_tiles(s, 32) * sizeof(int2)));
  v.bm = tile_bm(s);
  return v;
}

size_t ffn_ws_bytes(const Shape& s) {
  // schedule (at the smallest tile) + tile count + h [S][F]
  return align_up(max_tiles(s, 32) * sizeof(int2)) + align_up(sizeof(int)) +
         align_up((size_t)s.S * s.F * act_bytes(s));
}

hipError_t expert_ffn(const Shape& s, const void* x, const int32_t* sorted_slot,
                      const int32_t* offsets, const void* w_gate, const void* w_up,
                      const void* w_down, const float* s_gate, const float* s_up,
                      const float* s_down, const float* topk_w, void* y, void* ws,
                      hipStream_t st, bool schedule_ready, hipEvent_t const* ev) {
  if (s.S == 0) return hipSuccess;
  const FfnSchedule sv = ffn_schedule_view(s, ws);
  int2* tiles = sv.tiles;
  int* ntiles = sv.ntiles;
  uint16_t* h = reinterpret_cast<uint16_t*>(static_cast<unsigned char*>(ws) +
                                            align_up(max_tiles(s, 32) * sizeof(int2)) +
                                            align_up(sizeof(int)));
  const int bm = sv.bm;
  hipError_t e = hipSuccess;
  if (!schedule_ready) {
    hipLaunchKernelGGL(ffn_schedule_kernel, dim3(1), dim3(kMaxExperts), 0, st, offsets, s.El, bm,
                       tiles, ntiles);
    e = hipGetLastError();
  }
  if (e == hipSuccess && ev) e = hipEventRecord(ev[0], st);
  if (e != hipSuccess) return e;

  GemmArgs gu{};
  gu.A = static_cast<const uint16_t*>(x);
  gu.sorted_slot = sorted_slot;
  gu.k = s.k;
  gu.W0 = w_gate;
  gu.W1 = w_up;
  gu.S0 = s_gate;
  gu.S1 = s_up;
  gu.topk_w = nullptr;
  gu.out = h;
  gu.offsets = offsets;
  gu.tiles = tiles;
  gu.ntiles = ntiles;
  gu.K = s.d;
  gu.Nout = s.F;

  GemmArgs dn = gu;
  dn.A = h;
  dn.W0 = w_down;
  dn.W1 = nullptr;
  dn.S0 = s_down;
  dn.S1 = nullptr;
  dn.topk_w = topk_w;
  dn.out = static_cast<uint16_t*>(y);
  dn.K = s.F;
  dn.Nout = s.d;

  const long long mt = (long long)max_tiles(s, bm);
  if (s.weight == kF32) {
    gu.n_tiles_n = (s.F + kF32BN - 1) / kF32BN;
    dn.n_tiles_n = (s.d + kF32BN - 1) / kF32BN;
    const int grid = 4 * num_cu();
    hipLaunchKernelGGL(grouped_f32_kernel<true>, dim3(grid), dim3(256), 0, st, gu);
    e = hipGetLastError();
    if (e == hipSuccess && ev) e = hipEventRecord(ev[1], st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(grouped_f32_kernel<false>, dim3(grid), dim3(256), 0, st, dn);
    e = hipGetLastError();
    if (e == hipSuccess && ev) e = hipEventRecord(ev[2], st);
    return e;
  }
  const bool fp8 = s.weight == kFP8;
  if (use_decode_tiles(s)) {
    // 32 rows x 256 weight rows, 4 waves side by side along N
    gu.n_tiles_n = s.F / 128;
    dn.n_tiles_n = (s.d + 255) / 256;
    if (fp8) {
      e = launch_gemm<1, 1, 2, 4, true, true, 2>(gu, mt * gu.n_tiles_n, st);
      if (e == hipSuccess && ev) e = hipEventRecord(ev[1], st);
      if (e == hipSuccess) e = launch_gemm<1, 1, 2, 4, false, true, 2>(dn, mt * dn.n_tiles_n, st);
    } else {
      e = launch_gemm<1, 1, 2, 4, true, false, 2>(gu, mt * gu.n_tiles_n, st);
      if (e == hipSuccess && ev) e = hipEventRecord(ev[1], st);
      if (e == hipSuccess) e = launch_gemm<1, 1, 2, 4, false, false, 2>(dn, mt * dn.n_tiles_n, st);
    }
  } else {
    // 128 rows x 256 weight rows, 2 x 2 waves of 64 x 128
    gu.n_tiles_n = s.F / 128;
    dn.n_tiles_n = (s.d + 255) / 256;
    if (fp8) {
      e = launch_gemm<2, 2, 4, 2, true, true, 1>(gu, mt * gu.n_tiles_n, st);
      if (e == hipSuccess && ev) e = hipEventRecord(ev[1], st);
      if (e == hipSuccess) e = launch_gemm<2, 2, 4, 2, false, true, 1>(dn, mt * dn.n_tiles_n, st);
    } else {
      e = launch_gemm<2, 2, 4, 2, true, false, 1>(gu, mt * gu.n_tiles_n, st);
      if (e == hipSuccess && ev) e = hipEventRecord(ev[1], st);
      if (e == hipSuccess) e = launch_gemm<2, 2, 4, 2, false, false, 1>(dn, mt * dn.n_tiles_n, st);
    }
  }
  if (e == hipSuccess && ev) e = hipEventRecord(ev[2], st);
  return e;
}

}  // namespace moe
