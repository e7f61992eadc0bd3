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
  int group_m;                 // M tiles per rasterization group (>= 1)
};

// ---- LDS layout of the pipeline stages
// A stage holds BM rows of kBK bf16 activations and BNW weight rows of kBK K
// values (bf16, or one byte per FP8 code).  Rows are cut into 16-byte chunks;
// chunk c of row r sits at physical chunk c ^ swz(r).  The LDS serves a
// 16-byte read for 16 lanes per cycle over 64 banks (256 B), and an MFMA
// operand read has those 16 lanes on 16 consecutive rows at one logical
// chunk.  With R = 256 / row bytes rows per bank sweep and C chunks per row
// (R * C = 16), swz(r) = (r / R) % C gives the 16 lanes 16 distinct bank
// groups: r % R picks the sweep slot, r / R the chunk.
template <int kRowBytes>
__device__ __forceinline__ int lds_off(int r, int c) {
  constexpr int C = kRowBytes / 16;
  constexpr int R = 256 / kRowBytes;
  static_assert(R * C == 16, "row size");
  return r * kRowBytes + ((c ^ ((r / R) % C)) << 4);
}

// s_waitcnt that waits until at most N vector-memory operations of this wave
// (loads, stores, LDS-DMA loads) are outstanding; LGKM and EXP are left alone
// (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Scheduling hint for one MFMA step: kReads LDS reads alternating with the
// first kReads of the step's kMfma MFMAs, then the remaining MFMAs.
template <int kReads, int kMfma>
__device__ __forceinline__ void sched_alternate() {
  constexpr int kPairs = kReads < kMfma ? kReads : kMfma;
#pragma unroll
  for (int q = 0; q < kPairs; ++q) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
  }
  if constexpr (kMfma > kPairs) __builtin_amdgcn_sched_group_barrier(0x008, kMfma - kPairs, 0);
  if constexpr (kReads > kPairs) __builtin_amdgcn_sched_group_barrier(0x100, kReads - kPairs, 0);
}

// s_waitcnt lgkmcnt(0): this wave's LDS reads have returned (vmcnt and
// expcnt left alone).
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Workgroup barrier without a memory fence.  LDS-DMA data of a stage is in
// LDS once the issuing wave's vmcnt wait returns, and LDS executes each
// wave's operations in order; the empty asm statements keep the compiler from
// moving memory accesses across the barrier.  (__syncthreads would add a
// fence that waits for every load in flight, i.e. for all later stages too.)
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One 16-byte global -> LDS load per lane (gfx950 global_load_lds_dwordx4):
// lane i's 16 bytes land at lds + 16 i; `lds` must be wave-uniform.  The body
// exists only in the device pass (the host pass never runs it, and clang
// drops the host launch stubs of kernels that name this builtin directly).
__device__ __forceinline__ void lds_dma16(const void* src, unsigned char* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
#else
  (void)src;
  (void)lds;
#endif
}

template <int MB, int WM, int NB, int WN, bool kGateUp, bool kFP8, int kBK, int kStages>
struct Cfg {
  static constexpr int kWaves = WM * WN;
  static constexpr int kThreads = kWave * kWaves;
  static constexpr int BM = 32 * MB * WM;    // tile rows
  static constexpr int BNW = 32 * NB * WN;   // weight rows per tile
  static constexpr int kRowA = kBK * 2;      // bytes per A row per stage
  static constexpr int kRowB = kBK * (kFP8 ? 1 : 2);
  static constexpr int kChunksA = kRowA / 16;
  static constexpr int kChunksB = kRowB / 16;
  static constexpr int kStageA = BM * kRowA;
  static constexpr int kStageB = BNW * kRowB;
  static constexpr int kStage = kStageA + kStageB;
  static constexpr int kLoadsA = kStageA / (1024 * kWaves);  // 1 KB LDS-DMA loads per wave
  static constexpr int kLoadsB = kStageB / (1024 * kWaves);
  static constexpr int kLoads = kLoadsA + kLoadsB;
  static constexpr int kSteps = kBK / 16;                     // MFMA K steps per stage
  static constexpr int kScaleSets = kFP8 ? (kGateUp ? 2 : BNW / 128) : 0;
  static constexpr int kMaxKBlocks = 65536 / 128;
  static constexpr int kLds = kStages * kStage + kScaleSets * kMaxKBlocks * 4;
  static_assert(kBK == 32 || kBK == 64, "K step");
  static_assert(kStageA % (1024 * kWaves) == 0 && kStageB % (1024 * kWaves) == 0, "load split");
  static_assert(!kGateUp || NB % 2 == 0, "gate/up pairs column blocks");
  static_assert(kStages >= 2 && (kStages - 1) * kLoads < 64, "vmcnt budget");
  static_assert(kLds <= 160 * 1024, "LDS budget");
  static_assert(128 % kBK == 0, "a scale block spans whole K steps");
  static_assert(!kFP8 || !kGateUp || BNW / 2 == 128, "gate/up scales: one 128-row block");
  static_assert(!kFP8 || BNW % 128 == 0, "down scales: whole 128-row blocks");
  static_assert(!kFP8 || kBK == 64, "FP8 raw codes are double-buffered per step pair");
  static_assert(kSteps % 2 == 0, "fragment buffers alternate by step");
};

template <int MB, int WM, int NB, int WN, bool kGateUp, bool kFP8, int kBK, int kStages,
          int kMinBlocks>
__global__ __launch_bounds__(kWave* WM* WN, kMinBlocks) void grouped_gemm_kernel(GemmArgs a) {
  using C = Cfg<MB, WM, NB, WN, kGateUp, kFP8, kBK, kStages>;
  constexpr int BNW = C::BNW;
  constexpr int H = NB / 2;  // gate/up: column blocks per half
  extern __shared__ __align__(16) unsigned char smem[];
  float* sc_lds = reinterpret_cast<float*>(smem + kStages * C::kStage);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int l = lane_id();
  const int g = l >> 5;  // which 8 of an MFMA step's 16 K values this lane holds
  const int wm = wave % WM;
  const int wn = wave / WM;
  const int welem = kFP8 ? 1 : 2;  // bytes per weight element
  const int nK = a.K / kBK;
  const int KB = a.K / 128;

  // persistent, XCD-contiguous item ranges
  const int n_items = *a.ntiles * a.n_tiles_n;
  const int xcd = blockIdx.x % kNumXcd;
  const int per_xcd = gridDim.x / kNumXcd;
  const int slot = blockIdx.x / kNumXcd;
  const int it_begin = (int)((long long)n_items * xcd / kNumXcd);
  const int it_end = (int)((long long)n_items * (xcd + 1) / kNumXcd);

  // weight-tile row of this lane's MFMA column in block n
  auto brow = [&](int n) -> int {
    if (kGateUp) return (n < H ? 0 : BNW / 2) + wn * H * 32 + (n % H) * 32 + (l & 31);
    return wn * NB * 32 + n * 32 + (l & 31);
  };
  const int arow_base = wm * MB * 32 + (l & 31);

  const int n_mtiles = *a.ntiles;
  for (int item = it_begin + slot; item < it_end; item += per_xcd) {
    // grouped order: items run through groups of group_m consecutive M tiles,
    // M fastest inside a group, so the workgroups of an XCD that run at the
    // same time share a few A tiles and a few weight tiles in L2 (instead of
    // one A tile and as many weight tiles as workgroups)
    const int per_group = a.group_m * a.n_tiles_n;
    const int grp = item / per_group;
    const int first_m = grp * a.group_m;
    const int gsize = min(a.group_m, n_mtiles - first_m);
    const int in_grp = item - grp * per_group;
    const int gt = first_m + in_grp % gsize;
    const int nt = in_grp / gsize;
    const int2 tile = a.tiles[gt];
    const int j = tile.x;
    const int row0 = tile.y;
    const int row_end = a.offsets[j + 1];
    const int n0 = nt * (kGateUp ? BNW / 2 : BNW);  // first output column of the tile

    // ---- this lane's source chunk of every LDS-DMA load of a stage (step 0)
    const unsigned char* srcA[C::kLoadsA];
#pragma unroll
    for (int i = 0; i < C::kLoadsA; ++i) {
      const int P = (wave * C::kLoadsA + i) * kWave + l;  // 16-byte chunk position
      const int r = P / C::kChunksA;
      const int c = (P % C::kChunksA) ^ ((r / (256 / C::kRowA)) % C::kChunksA);
      const int p = min(row0 + r, row_end - 1);
      const long long arow = kGateUp ? (long long)(a.sorted_slot[p] / a.k) : (long long)p;
      srcA[i] = reinterpret_cast<const unsigned char*>(a.A + arow * a.K) + c * 16;
    }
    const unsigned char* srcB[C::kLoadsB];
#pragma unroll
    for (int i = 0; i < C::kLoadsB; ++i) {
      const int P = (wave * C::kLoadsB + i) * kWave + l;
      const int r = P / C::kChunksB;
      const int c = (P % C::kChunksB) ^ ((r / (256 / C::kRowB)) % C::kChunksB);
      const unsigned char* base;
      int wrow;
      if (kGateUp) {
        const bool up = r >= BNW / 2;
        wrow = min(n0 + (up ? r - BNW / 2 : r), a.Nout - 1);
        base = static_cast<const unsigned char*>(up ? a.W1 : a.W0);
      } else {
        wrow = min(n0 + r, a.Nout - 1);
        base = static_cast<const unsigned char*>(a.W0);
      }
      srcB[i] = base + ((long long)j * a.Nout + wrow) * a.K * welem + c * 16;
    }

    stage_barrier();  // every wave is done with the previous item's stages and scales
    if constexpr (kFP8) {
      // this tile's block scales -> LDS: set sb holds gate/up (gate/up GEMM) or
      // the sb-th 128-row block of the tile (down GEMM), for every K block
      for (int o = tid; o < C::kScaleSets * KB; o += C::kThreads) {
        const int sb = o / KB, kb = o % KB;
        const float* S = (kGateUp && sb == 1) ? a.S1 : a.S0;
        const int nblk = min(kGateUp ? n0 / 128 : n0 / 128 + sb, a.Nout / 128 - 1);
        sc_lds[sb * C::kMaxKBlocks + kb] = S[((long long)j * (a.Nout / 128) + nblk) * KB + kb];
      }
    }

#define MOE_ISSUE_STAGE(KS)                                                                     \
  do {                                                                                          \
    unsigned char* sb_ = smem + ((KS) % kStages) * C::kStage;                                   \
    _Pragma("unroll") for (int i = 0; i < C::kLoadsA; ++i)                                      \
        lds_dma16(srcA[i] + (long long)(KS) * kBK * 2, sb_ + (wave * C::kLoadsA + i) * 1024);   \
    _Pragma("unroll") for (int i = 0; i < C::kLoadsB; ++i)                                      \
        lds_dma16(srcB[i] + (long long)(KS) * kBK * welem,                                      \
                  sb_ + C::kStageA + (wave * C::kLoadsB + i) * 1024);                            \
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

    // MFMA operand fragments of one K step (tokens: A; weights: B; FP8
    // weights as raw codes for a pair of steps, widened at use).  K
    // permutation shared by both operands: bf16 weights use chunk 2s + g at
    // step s; an FP8 lane holds one 16-byte chunk (16 K values) for steps
    // 2p and 2p + 1.
    bf16x8_t af[2][MB];
    bf16x8_t bf[2][kFP8 ? 1 : NB];
    u32x4_t raw8[2][kFP8 ? NB : 1];
    auto read_frags = [&](int stage, int s, int buf) {
      const unsigned char* As = smem + (stage % kStages) * C::kStage;
      const unsigned char* Bs = As + C::kStageA;
      const int cA = kFP8 ? (4 * (s >> 1) + 2 * g + (s & 1)) : (2 * s + g);
#pragma unroll
      for (int m = 0; m < MB; ++m)
        af[buf][m] = *reinterpret_cast<const bf16x8_t*>(
            As + lds_off<C::kRowA>(arow_base + m * 32, cA));
      if constexpr (kFP8) {
        if ((s & 1) == 0) {
#pragma unroll
          for (int n = 0; n < NB; ++n)
            raw8[(s >> 1) & 1][n] = *reinterpret_cast<const u32x4_t*>(
                Bs + lds_off<C::kRowB>(brow(n), 2 * (s >> 1) + g));
        }
      } else {
#pragma unroll
        for (int n = 0; n < NB; ++n)
          bf[buf][n] = *reinterpret_cast<const bf16x8_t*>(
              Bs + lds_off<C::kRowB>(brow(n), 2 * s + g));
      }
    };
    auto mfma_step = [&](int s, int buf) {
#pragma unroll
      for (int n = 0; n < NB; ++n) {
        bf16x8_t bfr;
        if constexpr (kFP8) {
          const u32x4_t r = raw8[(s >> 1) & 1][n];
          const u32x2_t lo = e4m3x4_to_bf16x4(r[(s & 1) * 2]);
          const u32x2_t hi = e4m3x4_to_bf16x4(r[(s & 1) * 2 + 1]);
          bfr = __builtin_bit_cast(bf16x8_t, u32x4_t{lo.x, lo.y, hi.x, hi.y});
        } else {
          bfr = bf[buf][n];
        }
#pragma unroll
        for (int m = 0; m < MB; ++m) {
          // weights as the MFMA A operand: the result block is [feature][token]
          if constexpr (kFP8)
            part[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr, af[buf][m], part[m][n], 0, 0, 0);
          else
            acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr, af[buf][m], acc[m][n], 0, 0, 0);
        }
      }
    };

    // prologue: all stages in flight, stage 0 landed, its first fragments read
#pragma unroll
    for (int st = 0; st < kStages; ++st)
      if (st < nK) MOE_ISSUE_STAGE(st);
    if (nK >= kStages)
      wait_vmcnt<(kStages - 1) * C::kLoads>();
    else
      wait_vmcnt<0>();
    stage_barrier();
    read_frags(0, 0, 0);

    // Steady state.  The barrier for stage ks + 1 sits between the last two
    // MFMA steps of stage ks: waves wait at it while their earlier MFMAs still
    // occupy the matrix pipe, then refill the freed buffer of stage ks with
    // stage ks + kStages and read stage ks + 1's first fragments while the
    // last step's MFMAs run.
    for (int ks = 0; ks < nK; ++ks) {
#pragma unroll
      for (int s = 0; s < C::kSteps; ++s) {
        if (s + 1 < C::kSteps) {
          read_frags(ks, s + 1, (s + 1) & 1);
          mfma_step(s, s & 1);
          // alternate MFMA and LDS read (the next step's fragments): bursts of
          // reads stall the issuing waves, alternating keeps the matrix pipe fed
          if (kFP8 && (s + 1) % 2 != 0)  // FP8 weights are read every other step
            sched_alternate<MB, MB * NB>();
          else
            sched_alternate<MB + NB, MB * NB>();
        } else {
          __builtin_amdgcn_sched_barrier(0);
          wait_lgkmcnt0();  // this wave's reads of stage ks have returned
          if (ks + 1 < nK) {
            if (ks + kStages - 1 < nK)
              wait_vmcnt<(kStages - 2) * C::kLoads>();  // stage ks + 1 landed
            else
              wait_vmcnt<0>();
          }
          stage_barrier();  // stage ks + 1 visible; nobody reads stage ks any more
          if (ks + kStages < nK) MOE_ISSUE_STAGE(ks + kStages);
          __builtin_amdgcn_sched_barrier(0);
          if (ks + 1 < nK) read_frags(ks + 1, 0, 0);
          mfma_step(s, s & 1);
          if (ks + 1 < nK) sched_alternate<MB + NB, MB * NB>();
        }
      }
      if constexpr (kFP8) {
        if ((ks + 1) % (128 / kBK) == 0) {  // end of a 128-deep scale block
          const int kb = (ks * kBK) / 128;
          float sc[NB];
#pragma unroll
          for (int n = 0; n < NB; ++n) {
            const int sb = kGateUp ? (n < H ? 0 : 1) : (wn * NB * 32 + n * 32) / 128;
            sc[n] = sc_lds[sb * C::kMaxKBlocks + kb];
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
    }
#undef MOE_ISSUE_STAGE

    // ---- epilogue.  Each result block is [feature][token] (MFMA 32x32 layout:
    // lane l holds token column l % 32 and features 8 (q / 4) + 4 (l / 32) +
    // (q % 4) for register q), so a lane owns runs of 4 consecutive features
    // of one token row: one 8-byte store per run.
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      const int p = row0 + wm * MB * 32 + m * 32 + (l & 31);
      if (p < row_end) {
        uint16_t* orow = a.out + (long long)p * a.Nout;
        if constexpr (kGateUp) {
#pragma unroll
          for (int n = 0; n < H; ++n) {
#pragma unroll
            for (int q = 0; q < 16; q += 4) {
              const int col = n0 + wn * H * 32 + n * 32 + 8 * (q >> 2) + 4 * (l >> 5);
              if (col < a.Nout) {
                float h[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) h[u] = silu_f32(acc[m][n][q + u]) * acc[m][n + H][q + u];
                *reinterpret_cast<u32x2_t*>(orow + col) =
                    u32x2_t{pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3])};
              }
            }
          }
        } else {
          const float gw = a.topk_w ? a.topk_w[a.sorted_slot[p]] : 1.0f;
#pragma unroll
          for (int n = 0; n < NB; ++n) {
#pragma unroll
            for (int q = 0; q < 16; q += 4) {
              const int col = n0 + wn * NB * 32 + n * 32 + 8 * (q >> 2) + 4 * (l >> 5);
              if (col < a.Nout)
                *reinterpret_cast<u32x2_t*>(orow + col) =
                    u32x2_t{pack_bf16x2(acc[m][n][q] * gw, acc[m][n][q + 1] * gw),
                            pack_bf16x2(acc[m][n][q + 2] * gw, acc[m][n][q + 3] * gw)};
            }
          }
        }
      }
    }
  }
}

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

template <int MB, int WM, int NB, int WN, bool kGateUp, bool kFP8, int kBK, int kStages,
          int kMinBlocks>
hipError_t launch_gemm(const GemmArgs& a, long long max_items, hipStream_t st) {
  using C = Cfg<MB, WM, NB, WN, kGateUp, kFP8, kBK, kStages>;
  auto kern = grouped_gemm_kernel<MB, WM, NB, WN, kGateUp, kFP8, kBK, kStages, kMinBlocks>;
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

// Tile plans.  Decode (a handful of rows per expert): 32 x 256 tiles, four
// waves side by side along N, 64-deep K steps, 4 stages.  bf16 prefill: eight
// waves of 64 x 128, 32-deep K steps and 4 stages, as 128 x 512 tiles when
// experts hold a few hundred rows (less M padding) or 256 x 256 when they hold
// a thousand or more (fewer bytes staged per MFMA).  FP8 weights: four waves
// (each keeps a second accumulator set for the per-block scales), 128 x 256
// tiles, 64-deep K steps and 4 stages.
enum class Plan { kF32, kDecode, kWide, kBig, kFp8 };

Plan plan_of(const Shape& s) {
  if (s.weight == kF32) return Plan::kF32;
  if (s.S <= 64LL * s.El) return Plan::kDecode;
  if (s.weight == kFP8) return Plan::kFp8;
  return s.S >= 1024LL * s.El ? Plan::kBig : Plan::kWide;
}

bool use_decode_tiles(const Shape& s) { return plan_of(s) == Plan::kDecode; }

int tile_bm(const Shape& s) {
  switch (plan_of(s)) {
    case Plan::kF32: return kF32BM;
    case Plan::kDecode: return 32;
    case Plan::kBig: return 256;
    default: return 128;
  }
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
  // decode tiles (about one M tile per expert) gain nothing from grouping and
  // stream best in plain M-major order; prefill tiles group 8 M tiles
  gu.group_m = dn.group_m = use_decode_tiles(s) ? 1 : 8;
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
  auto ntn = [](int cols, int per_tile) { return (cols + per_tile - 1) / per_tile; };
  switch (plan_of(s)) {
    case Plan::kDecode:
      gu.n_tiles_n = ntn(s.F, 128);
      dn.n_tiles_n = ntn(s.d, 256);
      if (fp8) {
        e = launch_gemm<1, 1, 2, 4, true, true, 64, 4, 2>(gu, mt * gu.n_tiles_n, st);
        if (e == hipSuccess && ev) e = hipEventRecord(ev[1], st);
        if (e == hipSuccess) e = launch_gemm<1, 1, 2, 4, false, true, 64, 4, 2>(dn, mt * dn.n_tiles_n, st);
      } else {
        e = launch_gemm<1, 1, 2, 4, true, false, 64, 4, 1>(gu, mt * gu.n_tiles_n, st);
        if (e == hipSuccess && ev) e = hipEventRecord(ev[1], st);
        if (e == hipSuccess) e = launch_gemm<1, 1, 2, 4, false, false, 64, 4, 1>(dn, mt * dn.n_tiles_n, st);
      }
      break;
    case Plan::kFp8:
      gu.n_tiles_n = ntn(s.F, 128);
      dn.n_tiles_n = ntn(s.d, 256);
      e = launch_gemm<2, 2, 4, 2, true, true, 64, 4, 1>(gu, mt * gu.n_tiles_n, st);
      if (e == hipSuccess && ev) e = hipEventRecord(ev[1], st);
      if (e == hipSuccess) e = launch_gemm<2, 2, 4, 2, false, true, 64, 4, 1>(dn, mt * dn.n_tiles_n, st);
      break;
    case Plan::kWide:
      gu.n_tiles_n = ntn(s.F, 256);
      dn.n_tiles_n = ntn(s.d, 512);
      e = launch_gemm<2, 2, 4, 4, true, false, 32, 4, 1>(gu, mt * gu.n_tiles_n, st);
      if (e == hipSuccess && ev) e = hipEventRecord(ev[1], st);
      if (e == hipSuccess) e = launch_gemm<2, 2, 4, 4, false, false, 32, 4, 1>(dn, mt * dn.n_tiles_n, st);
      break;
    case Plan::kBig:
      gu.n_tiles_n = ntn(s.F, 128);
      dn.n_tiles_n = ntn(s.d, 256);
      e = launch_gemm<2, 4, 4, 2, true, false, 32, 4, 1>(gu, mt * gu.n_tiles_n, st);
      if (e == hipSuccess && ev) e = hipEventRecord(ev[1], st);
      if (e == hipSuccess) e = launch_gemm<2, 4, 4, 2, false, false, 32, 4, 1>(dn, mt * dn.n_tiles_n, st);
      break;
    case Plan::kF32:
      break;
  }
  if (e == hipSuccess && ev) e = hipEventRecord(ev[2], st);
  return e;
}

}  // namespace moe
