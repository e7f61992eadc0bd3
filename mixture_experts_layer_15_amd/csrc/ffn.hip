// Local experts: each expert's SwiGLU feed-forward network as a grouped GEMM
// over the ragged per-expert row segments of the dispatch order.
//
// "Serving MoE models with expert parallelism on 8xH200" (reviosa), section
// "Tensor parallel vs expert parallel": a GPU that owns whole experts runs
// full-size expert GEMMs on the tokens sent to it.  Section "Batching: MoE
// needs bigger batches than you think": at decode batch sizes each expert sees
// a handful of tokens and the expert GEMM only streams its weights from HBM;
// prefill gives each expert many rows.  Both regimes use the kernels below,
// with 32- or 64-row tiles for the first and 128- or 256-row tiles for the
// second.
//
//   gate/up:  h[p] = silu(A_p Wg_j) * (A_p Wu_j),  A_p = x[sorted_slot[p] / k]
//   down:     y[p] = (h[p] Wd_j) * gate(p)
//
// Structure (bf16 activations; bf16 or FP8-E4M3 weights):
//  * the permutation (or a one-workgroup schedule kernel) splits every expert
//    segment into M tiles of BM rows: (expert, first row, end row) per tile;
//  * a persistent GEMM kernel walks items (M tile, N tile); the items are cut
//    into eight contiguous ranges, one per XCD (workgroup b runs on XCD b % 8),
//    so items that share an A tile or a weight tile meet in the same L2;
//  * per item, a K loop over a ring of LDS stages filled by LDS-DMA (buffer
//    loads straight into LDS; A rows gathered through sorted_slot, weight rows
//    streamed; 16-byte chunks XOR-swizzled by row for the 64 LDS banks) ->
//    MFMA 32x32x16 bf16 with float32 accumulation, weights as the A operand;
//  * FP8 weights: raw codes through LDS, widened exactly to bf16 at use, and
//    a float32 scale per 128x128 block folded in by rescaling the accumulator
//    at each 128-deep K block, so the weights enter MFMA unrounded;
//  * MXFP4 weights ("Serving MoE models with expert parallelism on 8xH200",
//    sections "Memory math for 8xH200" and "Quantization choices"): E2M1
//    codes and their E8M0 block scales through LDS, each lane's 32 codes of a
//    stage widened to bf16 with the scale applied in one exact conversion;
//  * epilogues: silu(gate) * up rounded to bf16 (gate/up), or the product
//    times the token's gate (down).
#include <stdlib.h>

#include <algorithm>
#include <atomic>
#include <type_traits>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kNumXcd = 8;

__global__ __launch_bounds__(kMaxExperts) void ffn_schedule_kernel(const int32_t* offsets, int El,
                                                                   int BM, int4* tiles,
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
  for (int i = 0; i < nt; ++i) tiles[first + i] = make_int4(e, lo + i * BM, lo + cnt, 0);
  if (e == El - 1) *ntiles = sums[e];
}

struct GemmArgs {
  const uint16_t* A;           // gate/up: x [T][K]; down: h [S][K]  (bf16)
  uint32_t a_bytes;            // bytes of A (gate/up: x)
  const int32_t* sorted_slot;  // gate/up gather
  int k;                       // top-k (slot -> token)
  const void* W0;              // gate (gate/up) or down weights
  const void* W1;              // up weights (gate/up)
  const void* S0;              // scales for W0: FP8 float32 128x128 blocks, MXFP4 E8M0 bytes
  const void* S1;              // scales for W1
  const float* topk_w;         // down epilogue gates, or null
  uint16_t* out;               // gate/up: h [S][Nout]; down: y [S][Nout]
  float* out_f32;              // router: logits without bias [rows][Nout]
  int rows;                    // router: token rows (one segment, tiles of BM)
  const int32_t* offsets;      // [El + 1]
  const int4* tiles;           // (expert, first row, expert's end row, 0)
  const int* ntiles;
  int K;                       // reduction length
  int Nout;                    // output columns
  int n_tiles_n;               // N tiles per M tile
  int group_m;                 // M tiles per rasterization group (>= 1)
  int blocked;                 // W0/W1 in the blocked layout (units of 32 rows x 64 K)
  // wave-streamed GEMMs with the K range split (ksplit > 1): float32
  // partial products [ksplit][rows][Nout] (gate/up: gate columns, then up
  // columns), summed by split_reduce_kernel
  int ksplit;
  float* part;
  int part_rows;
  // prefill-sized tiles: virtual workers the items are dealt to (the
  // device's compute units, a multiple of 8, at most kMaxVW; 0: no tail
  // split) and the float32 partial sums of the split tail items
  int vw;
  float* tail;
};

// ---- Tail split (prefill-sized tiles)
// The items are dealt to vw virtual workers, one per compute unit: worker v
// (on XCD v % 8) runs fw = n_items / vw whole items from its XCD's
// contiguous range.  The rem = n_items % vw items of the last, partial wave
// would keep rem compute units busy for a whole item while the others idle;
// instead each is cut along K into s parts (at most vw / rem, each at least
// kMinPartStages K stages: a part pays an item's pipeline fill and a store of
// its partial sums), at most one part per worker.  The parts store float32
// partial sums; tail_reduce_kernel, launched after the GEMM, adds them in
// part order and runs the epilogue.  The cut depends on n_items, vw and K
// only, never on the grid, so results do not depend on the grid either.
constexpr int kMaxVW = 256;
constexpr int kMinPartStages = 8;
constexpr int kMaxParts = 16;
constexpr int kTailTileFloats = 256 * 256;  // accumulators of one prefill tile (BM x BNW)

struct TailPlan {
  int full;  // items in whole waves (a multiple of vw)
  int rem;   // items of the partial wave
  int s;     // parts per tail item (1: tail items run whole)
};

// align: K stages per part boundary (FP8: 2, whole 128-deep scale blocks)
__device__ __forceinline__ TailPlan tail_plan(int n_items, int vw, int nK, int align) {
  TailPlan t{n_items, 0, 1};
  if (vw < kNumXcd) return t;
  t.full = n_items / vw * vw;
  t.rem = n_items - t.full;
  if (t.rem > 0) {
    int s = min(vw / t.rem, min(nK / kMinPartStages, nK / align));
    t.s = max(min(s, kMaxParts), 1);
  }
  return t;
}

// first K stage of part q of s
__device__ __forceinline__ int part_begin(int q, int s, int nK, int align) {
  return (q * (nK / align) / s) * align;
}

// A unit of a workgroup's work: an item, its K stages [k0, k1), and the
// index of its partial-sum buffer (-1: a whole item, epilogue in place).
struct Unit {
  int item, k0, k1, u;
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

// Raw buffer resource over `bytes` bytes at `base` (wave-uniform): loads
// through it take a 32-bit per-lane offset, and offsets at or past `bytes`
// read zeros instead of faulting.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// One 16-byte buffer -> LDS load per lane (buffer_load_dwordx4 ... lds): lane
// i's 16 bytes, from voffset + soffset in the buffer, land at lds + 16 i.
__device__ __forceinline__ void lds_dma16_buf(__amdgpu_buffer_rsrc_t r, uint32_t voffset,
                                              uint32_t soffset, unsigned char* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16,
                                           voffset, soffset, 0, 0);
#else
  (void)r;
  (void)voffset;
  (void)soffset;
  (void)lds;
#endif
}

// The same with the nontemporal cache policy (gfx950 "nt"): for weights that
// are streamed once per step and not re-read by other tiles, so they do not
// displace the lines that are (measured on the Qwen3 decode step: gate/up
// 137.0 -> 129.4 us, down 71.5 -> 67.2 us; on prefill-sized tiles, whose
// weight tiles are re-read by several M tiles through L2, 6 % slower, so
// only the decode plans use it).
__device__ __forceinline__ void lds_dma16_buf_nt(__amdgpu_buffer_rsrc_t r, uint32_t voffset,
                                                 uint32_t soffset, unsigned char* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16,
                                           voffset, soffset, 0, 2);
#else
  (void)r;
  (void)voffset;
  (void)soffset;
  (void)lds;
#endif
}

// One 4-byte buffer -> LDS load per active lane (buffer_load_dword ... lds):
// lane i's 4 bytes, from voffset + soffset in the buffer, land at lds + 4 i.
__device__ __forceinline__ void lds_dma4_buf(__amdgpu_buffer_rsrc_t r, uint32_t voffset,
                                             uint32_t soffset, unsigned char* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 4,
                                           voffset, soffset, 0, 0);
#else
  (void)r;
  (void)voffset;
  (void)soffset;
  (void)lds;
#endif
}

// One 4-byte global -> LDS load per active lane (global_load_lds_dword): lane
// i's value lands at lds + 4 i.
__device__ __forceinline__ void lds_dma4(const void* src, unsigned char* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds, 4, 0, 0);
#else
  (void)src;
  (void)lds;
#endif
}

// kWBits: weight bits, 16 (bf16), 8 (FP8 E4M3) or 4 (MXFP4 E2M1)
template <int MB, int WM, int NB, int WN, bool kGateUp, int kWBits, int kBK, int kStages>
struct Cfg {
  static constexpr bool kFP8 = kWBits == 8;
  static constexpr bool kFP4 = kWBits == 4;
  static constexpr int kWaves = WM * WN;
  static constexpr int kThreads = kWave * kWaves;
  static constexpr int BM = 32 * MB * WM;    // tile rows
  static constexpr int BNW = 32 * NB * WN;   // weight rows per tile
  static constexpr int kRowA = kBK * 2;      // bytes per A row per stage
  static constexpr int kRowB = kBK * kWBits / 8;
  static constexpr int kChunksA = kRowA / 16;
  static constexpr int kChunksB = kRowB / 16;
  static constexpr int kStageA = BM * kRowA;
  static constexpr int kStageB = BNW * kRowB;
  // MXFP4: the stage's E8M0 scales after its weights, [kBK / 32][BNW] bytes
  // (tile rows in feature order: gate/up: gate features, then up features)
  static constexpr int kStageS = kFP4 ? (kBK / 32) * BNW : 0;
  static constexpr int kStage = kStageA + kStageB + kStageS;
  static constexpr int kLoadsA = kStageA / (1024 * kWaves);  // 1 KB LDS-DMA loads per wave
  static constexpr int kLoadsB = kStageB / (1024 * kWaves);
  // MXFP4 scale loads: 4-byte LDS-DMAs of kScaleLanes lanes, each inside one
  // K block and one weight matrix of the tile, kLoadsS per wave
  static constexpr int kScaleHalf = kGateUp ? BNW / 2 : BNW;  // bytes of one matrix per K block
  static constexpr int kScaleLanes =
      !kFP4 ? 1
            : (kScaleHalf / 4 < kWave ? kScaleHalf / 4 : kWave) < kStageS / (4 * kWaves)
                  ? (kScaleHalf / 4 < kWave ? kScaleHalf / 4 : kWave)
                  : kStageS / (4 * kWaves);
  static constexpr int kLoadsS = kFP4 ? kStageS / (4 * kScaleLanes * kWaves) : 0;
  static constexpr int kLoads = kLoadsA + kLoadsB + kLoadsS;
  static constexpr int kSteps = kBK / 16;                     // MFMA K steps per stage
  static constexpr int kScaleSets = kFP8 ? BNW / 128 : 0;  // 128-row weight blocks per tile
  static constexpr int kMaxKBlocks = 65536 / 128;
  static constexpr int kLds = kStages * kStage + 2 * kScaleSets * kMaxKBlocks * 4;
  static_assert(kBK == 32 || kBK == 64 || (kFP4 && kBK == 128), "K step");
  // MXFP4: 16-byte chunks (32 codes, one scale block) per lane, weight block
  // and stage; a lane covers K values g kBK/2 .. (g + 1) kBK/2 - 1 of a stage
  static constexpr int kFp4Chunks = kFP4 ? kBK / 64 : 1;
  static_assert(kStageA % (1024 * kWaves) == 0 && kStageB % (1024 * kWaves) == 0, "load split");
  static_assert(!kGateUp || NB % 2 == 0, "gate/up pairs column blocks");
  static_assert(kStages >= 2 && (kStages - 1) * kLoads < 64, "vmcnt budget");
  static_assert(kLds <= 160 * 1024, "LDS budget");
  static_assert(!kFP8 || 128 % kBK == 0, "a scale block spans whole K steps");
  static_assert(!kFP8 || (kGateUp ? (BNW / 2) % 128 == 0 : BNW % 128 == 0),
                "FP8 scales: whole 128-row weight blocks per tile (per half for gate/up)");
  static_assert(!kFP8 || kBK == 64, "FP8 raw codes are double-buffered per step pair");
  static_assert(!kFP4 || kBK == 64 || kBK == 128, "MXFP4: whole 32-value scale blocks per lane");
  static_assert(!kFP4 || (kScaleLanes >= 1 && kScaleLanes <= kWave && kLoadsS >= 1 &&
                          kStageS == 4 * kScaleLanes * kWaves * kLoadsS),
                "MXFP4 scales: whole dword LDS-DMAs per wave cover the stage's scales");
  static_assert(!kFP4 || kScaleHalf % (4 * kScaleLanes) == 0,
                "MXFP4 scales: one load's dwords lie in one K block and one weight matrix");
  static_assert(kSteps % 2 == 0, "fragment buffers alternate by step");
};

// item -> (M tile, first output column).  Grouped order: items run through
// groups of group_m consecutive M tiles, M fastest inside a group, so the
// workgroups of an XCD that run at the same time share a few A tiles and a
// few weight tiles in L2 (instead of one A tile and as many weight tiles as
// workgroups).
__device__ __forceinline__ int2 place_item(int item, int group_m, int n_mtiles, int n_tiles_n,
                                           int cols_per_tile) {
  const int per_group = group_m * n_tiles_n;
  const int grp = item / per_group;
  const int first_m = grp * group_m;
  const int gsize = min(group_m, n_mtiles - first_m);
  const int in_grp = item - grp * per_group;
  return make_int2(first_m + in_grp % gsize, (in_grp / gsize) * cols_per_tile);
}

// Epilogue of one 32 x 32 result block of a wave.  Each result block is
// [feature][token] (MFMA 32x32 layout: lane l holds token column l % 32 in
// its 16 registers); with the weight-row permutation, register q is feature
// 16 (l / 32) + q of the block, so a lane stores 16 consecutive features of
// its token row p from column col: two 16-byte stores.  gate/up:
// silu(v) * up; down: v times the row's gate gw.
template <bool kGateUp>
__device__ __forceinline__ void store_block(const GemmArgs& a, const f32x16_t& v,
                                            const f32x16_t& up, int p, int col, float gw) {
  if (col < a.Nout) {
    uint16_t* orow = a.out + (long long)p * a.Nout;
    float h[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) h[q] = kGateUp ? silu_f32(v[q]) * up[q] : v[q] * gw;
    *reinterpret_cast<u32x4_t*>(orow + col) =
        u32x4_t{pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]), pack_bf16x2(h[4], h[5]),
                pack_bf16x2(h[6], h[7])};
    *reinterpret_cast<u32x4_t*>(orow + col + 8) =
        u32x4_t{pack_bf16x2(h[8], h[9]), pack_bf16x2(h[10], h[11]), pack_bf16x2(h[12], h[13]),
                pack_bf16x2(h[14], h[15])};
  }
}

// Epilogue of one wave's accumulators: blocks (m, n) of rows c0 + arow_base +
// 32 m (those before the segment end ce) and columns n0c + 32 (wn kOut + n) +
// 16 g; gate/up pairs block n with its up block n + NB / 2.
template <int MB, int NB, bool kGateUp>
__device__ __forceinline__ void store_tile_rows(const GemmArgs& a, const f32x16_t (&acc)[MB][NB],
                                                int c0, int ce, int n0c, int arow_base, int wn,
                                                int g, const float (&gw)[kGateUp ? 1 : MB]) {
  constexpr int kOut = kGateUp ? NB / 2 : NB;
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    const int p = c0 + arow_base + m * 32;
    if (p < ce) {
#pragma unroll
      for (int n = 0; n < kOut; ++n)
        store_block<kGateUp>(a, acc[m][n], acc[m][n + (kGateUp ? kOut : 0)], p,
                             n0c + wn * kOut * 32 + n * 32 + 16 * g, gw[kGateUp ? 0 : m]);
    }
  }
}

// Partial sums of a split tail item: wave w's accumulators as
// [w][m][n][r][lane] float4 (r: registers 4r .. 4r + 3), so that each store
// or load instruction of a wave covers 1 KB of consecutive bytes.
template <int MB, int NB>
__device__ __forceinline__ f32x4_t* partial_at(float* unit_buf, int wave, int l) {
  return reinterpret_cast<f32x4_t*>(unit_buf) + wave * (MB * NB * 4 * kWave) + l;
}

// kRouter: the router products x W_r as one segment of `rows` token rows,
// A = x read row by row, W0 = the router matrix stored [E][d], float32 output.
// kBlk: weights in the blocked layout (units of 32 rows x 64 K values, each
// the image of the MFMA operand loads of one wave: see pack_weights_kernel).
template <int MB, int WM, int NB, int WN, bool kGateUp, int kWBits, int kBK, int kStages,
          int kMinBlocks, bool kRouter, bool kBlk>
__global__ __launch_bounds__(kWave* WM* WN, kMinBlocks) void grouped_gemm_kernel(GemmArgs a) {
  using C = Cfg<MB, WM, NB, WN, kGateUp, kWBits, kBK, kStages>;
  static_assert(!kBlk || (kBK == 64 && !kRouter), "blocked units are 64 K deep");
  constexpr bool kFP8 = C::kFP8;
  constexpr bool kFP4 = C::kFP4;
  static_assert(kWBits == 16 || kFP8 || kFP4, "weight bits");
  static_assert(!kRouter || (!kGateUp && kWBits == 16), "router mode: plain bf16 GEMM");
  constexpr int BNW = C::BNW;
  constexpr int H = NB / 2;  // gate/up: column blocks per half
  extern __shared__ __align__(16) unsigned char smem[];
  // LDS: kStages pipeline stages | FP8 block scales of two items (the running
  // one and the next), [sets][KB] each
  float* sc_lds = reinterpret_cast<float*>(smem + kStages * C::kStage);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int l = lane_id();
  const int g = l >> 5;  // which 8 of an MFMA step's 16 K values this lane holds
  const int wm = wave % WM;
  const int wn = wave / WM;
  const int nK = a.K / kBK;
  const int KB = a.K / 128;
  const int n_sc = C::kScaleSets * KB;  // scale floats per item

  // persistent, XCD-contiguous item ranges
  const int n_mtiles = kRouter ? (a.rows + C::BM - 1) / C::BM : *a.ntiles;
  // tile gt as (expert, first row, segment end row)
  auto tile_at = [&](int gt, int opaque_zero) -> int4 {
    if constexpr (kRouter) return make_int4(0, gt * C::BM, a.rows, 0);
    return a.tiles[gt + opaque_zero];
  };
  const int n_items = n_mtiles * a.n_tiles_n;
  const int xcd = blockIdx.x % kNumXcd;
  const int per_xcd = gridDim.x / kNumXcd;
  const int slot = blockIdx.x / kNumXcd;
  auto place = [&](int item) -> int2 {
    return place_item(item, a.group_m, n_mtiles, a.n_tiles_n, kGateUp ? BNW / 2 : BNW);
  };

  // This workgroup's units, numbered 0 .. n_units - 1.  Without a tail
  // split the items are cut into eight contiguous ranges, one per XCD, and
  // workgroup slot j of an XCD runs items j, j + per_xcd, ... of its range.
  // With one (prefill-sized tiles, tail_plan), the same for the whole waves
  // of a.vw virtual workers, then the parts of the tail items.
  constexpr bool kTail = !kRouter && C::BM >= 128;
  constexpr int kAlign = kFP8 ? 128 / kBK : 1;
  static_assert(!kTail || C::BM * C::BNW <= kTailTileFloats, "tail partials of one tile");
  const int vw = kTail && a.vw >= kNumXcd ? a.vw : gridDim.x;
  const TailPlan tp = kTail ? tail_plan(n_items, vw, nK, kAlign) : TailPlan{n_items, 0, 1};
  // Virtual worker v sits on XCD x = v % 8 as its slot j = v / 8 of vw / 8.
  // Whole items: XCD x owns the contiguous range [x, x + 1) * full / 8, and
  // slot j runs items j, j + vw / 8, ... of it.  Tail units u (part u / rem
  // of tail item u % rem) are dealt to the XCDs in contiguous runs of
  // per_x, so that neighbouring tail items (which share A and weight tiles)
  // run on one XCD: slot j of XCD x runs unit x * per_x + j.  Workgroup b
  // runs the virtual workers b, b + G, ... (G = gridDim.x, a multiple of 8:
  // all on b's XCD, slots jb, jb + G / 8, ...).
  const int fw = tp.full / vw;                       // whole items per virtual worker
  const int nu = tp.rem * tp.s;                      // tail units (<= vw)
  const int per_x = (nu + kNumXcd - 1) / kNumXcd;    // tail units per XCD
  const int jb = (int)blockIdx.x / kNumXcd;          // b's slot; b's XCD is xcd
  const int gx = (int)gridDim.x / kNumXcd;           // workgroup slots per XCD
  const int jmax = max(0, min(per_x, nu - xcd * per_x));  // XCD's slots with a tail unit
  const int nv = jb < vw / kNumXcd ? (vw / kNumXcd - jb + gx - 1) / gx : 0;  // b's workers
  const int n1 = jb < jmax ? (jmax - jb + gx - 1) / gx : 0;  // ... with a tail unit
  // router mode: each tile's K range may be cut into a.ksplit parts, whose
  // float32 products go to separate planes (the top-k kernels add them in
  // part order); the plain XCD ranges then run over (part, item)
  const int rks = kRouter ? max(a.ksplit, 1) : 1;
  const int it_begin = (int)((long long)n_items * rks * xcd / kNumXcd);
  const int it_end = (int)((long long)n_items * rks * (xcd + 1) / kNumXcd);
  // Without a split (tp.s == 1) the items keep the plain XCD ranges: the
  // last partial wave then runs next to the items of the same M tiles on each
  // XCD (measured 2-4 % faster than dealing the tail items out separately).
  const bool split = kTail && tp.s > 1;
  const int n_units = split ? n1 * (fw + 1) + (nv - n1) * fw
                            : max(0, (it_end - it_begin - slot + per_xcd - 1) / per_xcd);
  auto unit = [&](int k) -> Unit {
    if (!split) {
      const int idx = it_begin + slot + k * per_xcd;
      if (kRouter && rks > 1) {
        const int q = idx / n_items;  // part q of every item, then part q + 1
        return Unit{idx % n_items, part_begin(q, rks, nK, 1), part_begin(q + 1, rks, nK, 1), q};
      }
      return Unit{idx, 0, nK, -1};
    } else {
      int vi, r;
      if (k < n1 * (fw + 1)) {
        vi = k / (fw + 1), r = k % (fw + 1);
      } else {
        const int kk = k - n1 * (fw + 1);
        vi = n1 + kk / fw, r = kk % fw;
      }
      const int j = jb + vi * gx;  // slot of the virtual worker on XCD xcd
      if (r < fw) return Unit{xcd * (tp.full / kNumXcd) + j + r * (vw / kNumXcd), 0, nK, -1};
      const int u = xcd * per_x + j;
      const int t = u % tp.rem, q = u / tp.rem;  // tail unit u: part q of tail item t
      return Unit{tp.full + t, part_begin(q, tp.s, nK, kAlign),
                  part_begin(q + 1, tp.s, nK, kAlign), u};
    }
  };

  // Weight rows enter each 32-row MFMA block permuted: block row 8a + 4g + b
  // (a, b < 4; g < 2) holds feature 16g + 4a + b, so that a lane's 16 result
  // registers are 16 consecutive output features (see the epilogue).
  auto feat_of_row = [](int r) -> int {
    return (r & ~31) | (((r >> 2) & 1) << 4) | (((r >> 3) & 3) << 2) | (r & 3);
  };
  // LDS row of this lane's MFMA operand in weight block n (A operand of MFMA)
  auto brow = [&](int n) -> int {
    if (kGateUp) return (n < H ? 0 : BNW / 2) + wn * H * 32 + (n % H) * 32 + (l & 31);
    return wn * NB * 32 + n * 32 + (l & 31);
  };
  const int arow_base = wm * MB * 32 + (l & 31);
  // FP8: scale set (128-row weight block of the tile) of weight block n
  auto sblk = [&](int n) -> int {
    if (kGateUp) return (n < H ? 0 : C::kScaleSets / 2) + (wn * H * 32 + (n % H) * 32) / 128;
    return (wn * NB * 32 + n * 32) / 128;
  };

  // rows: gate/up: sorted_slot of the A row of each of this lane's LDS-DMA
  // chunks; down: sorted_slot of this lane's epilogue rows (for the gates)
  constexpr int kRows = kGateUp ? C::kLoadsA : MB;
  auto load_rows = [&](int row0, int row_end, int* rows) {
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
      if (kGateUp) {
        const int P = (wave * C::kLoadsA + i) * kWave + l;
        rows[i] = a.sorted_slot[min(row0 + P / C::kChunksA, row_end - 1)];
      } else if (!kRouter) {
        const int p = row0 + arow_base + i * 32;
        rows[i] = p < row_end ? a.sorted_slot[p] : 0;
      } else {
        rows[i] = 0;
      }
    }
  };
  // FP8: an item's block scales go straight to LDS (LDS-DMA, 64 floats per
  // wave instruction), into the scale buffer the item will read
  auto dma_scales = [&](int j, int n0, int buf) {
    for (int c0 = wave * kWave; c0 < n_sc; c0 += C::kThreads) {
      const int o = c0 + l;
      if (o < n_sc) {
        // set sb: the tile's sb-th 128-row weight block (gate/up: gate blocks,
        // then up blocks)
        const int sb = o / KB, kb = o % KB;
        constexpr int kHalf = (kGateUp ? C::kScaleSets / 2 : C::kScaleSets) > 0
                                  ? (kGateUp ? C::kScaleSets / 2 : C::kScaleSets)
                                  : 1;  // (FP8 only)
        const float* S = static_cast<const float*>((kGateUp && sb >= kHalf) ? a.S1 : a.S0);
        const int nblk = min(n0 / 128 + sb % kHalf, a.Nout / 128 - 1);
        lds_dma4(S + ((long long)j * (a.Nout / 128) + nblk) * KB + kb,
                 reinterpret_cast<unsigned char*>(sc_lds + buf * n_sc + c0));
      }
    }
  };

  // Sources of an item's LDS-DMA loads: buffer resources (scalar registers)
  // and one 32-bit offset per lane and load (stage 0); a stage's K offset is
  // a scalar added at issue.  (The host limits x, and one expert's weight
  // matrix, to 4 GiB.)
  __amdgpu_buffer_rsrc_t rsA, rsB0, rsB1;  // A rows; gate or down weights; up weights
  uint32_t offA[C::kLoadsA];
  uint32_t offB[C::kLoadsB];
  __amdgpu_buffer_rsrc_t rsS[C::kLoadsS > 0 ? C::kLoadsS : 1];  // MXFP4 scale loads' matrices
  uint32_t offS[C::kLoadsS > 0 ? C::kLoadsS : 1];
  // weight instruction i of this wave reads up rows (one half of the tile)
  auto b_up = [&](int i) -> bool {
    return kGateUp && ((wave * C::kLoadsB + i) * kWave) / C::kChunksB >= BNW / 2;
  };
  // bf16 decode gate/up on row-major weights: each item starts its K loop at
  // its own stage (rotation by expert and N tile), so that the workgroups
  // streaming weights at the same time do not all read the same offset of
  // their rows (measured: 2 % faster; on blocked weights, whose stages are
  // contiguous runs, 3 % slower, and no gain on the other plans).  The
  // rotation is a function of the item only, so results do not depend on the
  // grid.
  constexpr bool kRotK = kGateUp && kWBits == 16 && C::BM <= 64 && !kRouter && !kBlk;
  // decode-sized tiles: each weight tile is read by one M tile, streamed nontemporal
  constexpr bool kNtW = C::BM <= 64 && !kRouter;
  int qrot = 0;
  // (tail parts: qrot is the part's first K stage, and the part's stages
  // never reach the wrap-around)
  auto set_src = [&](int j, int row0, int row_end, int n0, const int* rows, int k0) {
    j = __builtin_amdgcn_readfirstlane(j);
    if constexpr (kRotK) qrot = __builtin_amdgcn_readfirstlane((j * 3 + n0 / 32) % nK);
    if constexpr (kTail || kRouter) qrot = __builtin_amdgcn_readfirstlane(k0);
    row0 = __builtin_amdgcn_readfirstlane(row0);
    row_end = __builtin_amdgcn_readfirstlane(row_end);
    const uint32_t arow_bytes = (uint32_t)a.K * 2;
    rsA = kGateUp ? buffer_rsrc(a.A, a.a_bytes)
                  : buffer_rsrc(reinterpret_cast<const unsigned char*>(a.A) +
                                    (size_t)row0 * arow_bytes,
                                (uint32_t)(row_end - row0) * arow_bytes);
#pragma unroll
    for (int i = 0; i < C::kLoadsA; ++i) {
      const int P = (wave * C::kLoadsA + i) * kWave + l;  // 16-byte chunk position
      const int r = P / C::kChunksA;
      const int c = (P % C::kChunksA) ^ ((r / (256 / C::kRowA)) % C::kChunksA);
      const uint32_t arow = kGateUp ? (uint32_t)(rows[kGateUp ? i : 0] / a.k)
                                    : (uint32_t)min(r, row_end - 1 - row0);
      offA[i] = arow * arow_bytes + c * 16;
    }
    const uint32_t wrow_bytes = (uint32_t)a.K * kWBits / 8;
    const uint32_t wmat = (uint32_t)a.Nout * wrow_bytes;  // bytes of one expert's matrix
    rsB0 = buffer_rsrc(static_cast<const unsigned char*>(a.W0) + (size_t)j * wmat, wmat);
    rsB1 = kGateUp ? buffer_rsrc(static_cast<const unsigned char*>(a.W1) + (size_t)j * wmat, wmat)
                   : rsB0;
#pragma unroll
    for (int i = 0; i < C::kLoadsB; ++i) {
      const int P = (wave * C::kLoadsB + i) * kWave + l;
      const int r = P / C::kChunksB;
      const int c = (P % C::kChunksB) ^ ((r / (256 / C::kRowB)) % C::kChunksB);
      const int rr = (kGateUp && r >= BNW / 2) ? r - BNW / 2 : r;
      const uint32_t wrow = (uint32_t)min(n0 + feat_of_row(rr), a.Nout - 1);
      offB[i] = wrow * wrow_bytes + c * 16;
    }
    if constexpr (kBlk) {
      // blocked weights: a stage's image of 32-row block b is one contiguous
      // unit of 32 x kRowB bytes, so lane l of load i copies the bytes at the
      // same position of that unit; a row block spans all K stages
      constexpr uint32_t kUnit = 32u * C::kRowB;
      const uint32_t rb_bytes = (uint32_t)nK * kUnit;
#pragma unroll
      for (int i = 0; i < C::kLoadsB; ++i) {
        const uint32_t o = (uint32_t)((wave * C::kLoadsB + i) * 1024 + 16 * l);
        int b = (int)(o / kUnit);
        if (kGateUp && b >= BNW / 64) b -= BNW / 64;
        const int rb = min(n0 / 32 + b, a.Nout / 32 - 1);
        offB[i] = (uint32_t)rb * rb_bytes + o % kUnit;
      }
    }
    if constexpr (kFP4) {
      // scale load i of this wave: stage bytes [wb, wb + 4 kScaleLanes), inside
      // K block kb of the stage and one matrix (wave-uniform); lane l:
      // features fo .. fo + 3 of that matrix
      const uint32_t smat = (uint32_t)(a.K / 32) * a.Nout;  // bytes of one expert's scales
#pragma unroll
      for (int i = 0; i < C::kLoadsS; ++i) {
        const int wb = (wave * C::kLoadsS + i) * C::kScaleLanes * 4;
        const int kb = wb / BNW;
        const bool up = kGateUp && (wb % BNW) >= BNW / 2;
        const int fo = (wb % BNW) - (up ? BNW / 2 : 0) + 4 * l;
        rsS[i] = buffer_rsrc(
            static_cast<const unsigned char*>(up ? a.S1 : a.S0) + (size_t)j * smat, smat);
        offS[i] = (uint32_t)kb * a.Nout + (uint32_t)min(n0 + fo, a.Nout - 4);
      }
    }
  };

  // stage Q of the item set_src chose, into the buffer of pipeline stage G
#define MOE_ISSUE_STAGE(Q, G)                                                                   \
  do {                                                                                          \
    unsigned char* sb_ = smem + ((G) % kStages) * C::kStage;                                    \
    const int qq_ = ((Q) + qrot) >= nK ? (Q) + qrot - nK : (Q) + qrot;  /* rotated K stage */    \
    _Pragma("unroll") for (int i = 0; i < C::kLoadsA; ++i)                                      \
        lds_dma16_buf(rsA, offA[i], (uint32_t)(qq_) * kBK * 2,                                    \
                      sb_ + (wave * C::kLoadsA + i) * 1024);                                    \
    _Pragma("unroll") for (int i = 0; i < C::kLoadsB; ++i) {                                    \
      if constexpr (kNtW)                                                                       \
        lds_dma16_buf_nt(b_up(i) ? rsB1 : rsB0, offB[i], (uint32_t)(qq_) * bstage,               \
                         sb_ + C::kStageA + (wave * C::kLoadsB + i) * 1024);                    \
      else                                                                                      \
        lds_dma16_buf(b_up(i) ? rsB1 : rsB0, offB[i], (uint32_t)(qq_) * bstage,                  \
                      sb_ + C::kStageA + (wave * C::kLoadsB + i) * 1024);                       \
    }                                                                                           \
    if constexpr (kFP4) {                                                                       \
      _Pragma("unroll") for (int i = 0; i < C::kLoadsS; ++i)                                    \
        if (l < C::kScaleLanes)                                                                 \
          lds_dma4_buf(rsS[i], offS[i], (uint32_t)(qq_) * (kBK / 32) * a.Nout,                    \
                       sb_ + C::kStageA + C::kStageB +                                          \
                           (wave * C::kLoadsS + i) * C::kScaleLanes * 4);                       \
    }                                                                                           \
  } while (0)

  // weight bytes between consecutive K stages of one row
  constexpr uint32_t bstage = kBlk ? 32u * C::kRowB : (uint32_t)C::kRowB;

  if (n_units <= 0) return;
  int kc = 0;  // running unit
  Unit U = unit(0);

  // tiles as (expert, first row, end row) and first output column of the
  // running unit (c), the next (x) and the one after it (y)
  int cj, c0, ce, n0c, xj = 0, x0 = 0, xe = 1, n0x = 0;
  {
    const int2 pl = place(U.item);
    const int4 t = tile_at(pl.x, 0);
    cj = t.x, c0 = t.y, ce = t.z, n0c = pl.y;
  }
  if (n_units > 1) {
    const int2 pl = place(unit(1).item);
    const int4 t = tile_at(pl.x, 0);
    xj = t.x, x0 = t.y, xe = t.z, n0x = pl.y;
  }
  int rows_cur[kRows];
  load_rows(c0, ce, rows_cur);
  // Every register load above has landed before the loop: the loop's own
  // waits for them then fall on points where all earlier loads are known
  // complete, and the compiler places no wait of its own inside the loop.
  wait_vmcnt<0>();
  if constexpr (kFP8) dma_scales(cj, n0c, 0);  // lands before stage 0 does
  set_src(cj, c0, ce, n0c, rows_cur, U.k0);
#pragma unroll
  for (int st = 0; st < kStages; ++st)
    if (st < U.k1 - U.k0) MOE_ISSUE_STAGE(st, st);
  // MFMA operand fragments of one K step (tokens: B operand; weights: A
  // operand; FP8 weights as raw codes for a pair of steps, widened at use).
  // K permutation shared by both operands: bf16 weights use chunk 2s + g at
  // step s; an FP8 lane holds one 16-byte chunk (16 K values) for steps
  // 2p and 2p + 1.
  bf16x8_t af[2][MB];
  bf16x8_t bf[2][(kFP8 || kFP4) ? 1 : NB];
  u32x4_t raw8[2][kFP8 ? NB : 1];
  // MXFP4: one 16-byte chunk (32 codes: K values 32 g .. 32 g + 31 of the
  // stage) and its block scale per weight block, by stage parity; step s
  // uses codes 8 s .. 8 s + 7
  u32x4_t raw4[2][kFP4 ? NB : 1][C::kFp4Chunks];
  float sc4[2][kFP4 ? NB : 1][C::kFp4Chunks];
  // MXFP4: byte of this lane's weight row in a stage's scale block (feature
  // order inside the tile)
  auto srow = [&](int n) -> int {
    if (kGateUp) return (n < H ? 0 : BNW / 2) + feat_of_row(wn * H * 32 + (n % H) * 32 + (l & 31));
    return feat_of_row(wn * NB * 32 + n * 32 + (l & 31));
  };
  // LDS offset of this lane's 16-byte weight chunk q (chunk pair: K values
  // 16 q + 8 g .. + 8 of bf16, 32 q + 16 g .. + 16 of FP8, 32 g .. + 32 of
  // MXFP4) of weight block n in a stage: row-major weights sit as swizzled
  // rows, blocked ones as units of 1 KB operand loads (lane l at 16 l)
  auto b_off = [&](int n, int q) -> int {
    if constexpr (kBlk) return (brow(n) >> 5) * (32 * C::kRowB) + q * 1024 + 16 * l;
    return lds_off<C::kRowB>(brow(n), 2 * q + g);
  };
  auto read_frags = [&](int stage, int s, int buf) {
    const unsigned char* As = smem + (stage % kStages) * C::kStage;
    const unsigned char* Bs = As + C::kStageA;
    const int cA = kFP4   ? (g * (kBK / 16) + s)
                   : kFP8 ? (4 * (s >> 1) + 2 * g + (s & 1))
                          : (2 * s + g);
#pragma unroll
    for (int m = 0; m < MB; ++m)
      af[buf][m] = *reinterpret_cast<const bf16x8_t*>(
          As + lds_off<C::kRowA>(arow_base + m * 32, cA));
    if constexpr (kFP4) {
      if (s == 0) {
        const unsigned char* Ss = Bs + C::kStageB;
#pragma unroll
        for (int n = 0; n < NB; ++n) {
#pragma unroll
          for (int c = 0; c < C::kFp4Chunks; ++c) {
            const int q = g * C::kFp4Chunks + c;  // chunk of the row = scale block of the stage
            raw4[stage & 1][n][c] = *reinterpret_cast<const u32x4_t*>(
                Bs + (kBlk ? b_off(n, c) : lds_off<C::kRowB>(brow(n), q)));
            sc4[stage & 1][n][c] = e8m0_to_f32(Ss[q * BNW + srow(n)]);
          }
        }
      }
    } else if constexpr (kFP8) {
      if ((s & 1) == 0) {
#pragma unroll
        for (int n = 0; n < NB; ++n)
          raw8[(s >> 1) & 1][n] = *reinterpret_cast<const u32x4_t*>(Bs + b_off(n, s >> 1));
      }
    } else {
#pragma unroll
      for (int n = 0; n < NB; ++n)
        bf[buf][n] = *reinterpret_cast<const bf16x8_t*>(Bs + b_off(n, s));
    }
  };

  int base = 0;    // pipeline stage number of this item's stage 0
  int parity = 0;  // scale buffer of this item

  for (;;) {
    const bool has_next = kc + 1 < n_units;
    const bool has_nn = kc + 2 < n_units;
    const Unit X = has_next ? unit(kc + 1) : U;
    const int y_item = has_nn ? unit(kc + 2).item : 0;
    const int nKc = U.k1 - U.k0;  // K stages of this unit

    // this item's stage 0 has landed once only its later stages (and younger
    // loads or stores) remain in flight
    if (nKc >= kStages)
      wait_vmcnt<(kStages - 1) * C::kLoads>();
    else
      wait_vmcnt<0>();
    stage_barrier();  // stage 0 and this item's scales are visible to all waves
    read_frags(base, 0, 0);

    // down: this item's gates, read in its epilogue
    float gw[kGateUp ? 1 : MB];
    if constexpr (!kGateUp) {
#pragma unroll
      for (int m = 0; m < MB; ++m)
        gw[m] = (!kRouter && a.topk_w && c0 + arow_base + m * 32 < ce) ? a.topk_w[rows_cur[m]]
                                                                         : 1.0f;
    }

    // the next item's inputs and the tile of the item after it
    int yj = xj, y0 = x0, ye = xe, n0y = n0x;
    int rows_nxt[kRows];
    if (has_nn) n0y = place(y_item).y;
    if (has_next) {
      load_rows(x0, xe, rows_nxt);
      if (has_nn) {
        // an index the compiler cannot prove wave-uniform keeps the tile in
        // vector registers: moving a loaded value to scalar registers would
        // wait for it (and for every stage load in flight) right here
        int opaque_zero;
        asm volatile("v_mov_b32 %0, 0" : "=v"(opaque_zero));
        const int4 t = tile_at(place(y_item).x, opaque_zero);
        yj = t.x, y0 = t.y, ye = t.z;
      }
      // the other scale buffer was last read by the previous item
      if constexpr (kFP8) dma_scales(xj, n0x, parity ^ 1);
    }

    f32x16_t acc[MB][NB];
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int n = 0; n < NB; ++n) acc[m][n] = f32x16_t{};
    // FP8 block scales.  acc[.][n] holds the running sum divided by rsc[n],
    // the scale of the latest K block with a nonzero scale.  Entering a block
    // with scale s multiplies acc by rsc / s and makes s the reference, so the
    // MFMAs add the block's unscaled products (exact bf16 widenings of the
    // codes) straight into acc; the end multiplies by rsc.  A block whose
    // scale is 0 contributes nothing: its codes are masked to 0 (behind a
    // wave-uniform flag, so other blocks pay one scalar branch).
    float rsc[kFP8 ? NB : 1];
    bool zblk[kFP8 ? NB : 1];
    bool anyz = false;
    if constexpr (kFP8) {
#pragma unroll
      for (int n = 0; n < NB; ++n) rsc[n] = 1.0f, zblk[n] = false;
    }

    // sp: parity of the pipeline stage (MXFP4 fragments are kept per stage)
    auto mfma_step = [&](int s, int buf, int sp) {
#pragma unroll
      for (int n = 0; n < NB; ++n) {
        bf16x8_t bfr;
        if constexpr (kFP4) {
          bfr = e2m1x8_to_bf16x8(raw4[sp][n][s >> 2][s & 3], sc4[sp][n][s >> 2]);
        } else if constexpr (kFP8) {
          u32x4_t r = raw8[(s >> 1) & 1][n];
          if (anyz && zblk[n]) r = u32x4_t{0u, 0u, 0u, 0u};
          const u32x2_t lo = e4m3x4_to_bf16x4(r[(s & 1) * 2]);
          const u32x2_t hi = e4m3x4_to_bf16x4(r[(s & 1) * 2 + 1]);
          bfr = __builtin_bit_cast(bf16x8_t, u32x4_t{lo.x, lo.y, hi.x, hi.y});
        } else {
          bfr = bf[buf][n];
        }
#pragma unroll
        for (int m = 0; m < MB; ++m) {
          // weights as the MFMA A operand: the result block is [feature][token]
          acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr, af[buf][m], acc[m][n], 0, 0, 0);
        }
      }
    };

    // K loop.  The barrier for stage ks + 1 sits between the last two MFMA
    // steps of stage ks: waves wait at it while their earlier MFMAs still
    // occupy the matrix pipe, then refill the freed buffer of stage ks with
    // stage ks + kStages and read stage ks + 1's first fragments while the
    // last step's MFMAs run.
    for (int ks = 0; ks < nKc; ++ks) {
      if constexpr (kFP8) {
        if (((U.k0 + ks) * kBK) % 128 == 0) {  // entering a 128-deep scale block
          const int kb = ((U.k0 + ks) * kBK) / 128;
          anyz = false;
#pragma unroll
          for (int n = 0; n < NB; ++n) {
            const int bits = __builtin_amdgcn_readfirstlane(
                __float_as_int(sc_lds[parity * n_sc + sblk(n) * KB + kb]));
            zblk[n] = (bits & 0x7fffffff) == 0;
            anyz = anyz || zblk[n];
            if (!zblk[n]) {
              const float sv = __int_as_float(bits);
              if (ks > 0) {  // not the unit's first block
                const float ratio = rsc[n] / sv;
#pragma unroll
                for (int m = 0; m < MB; ++m) acc[m][n] *= ratio;
              }
              rsc[n] = sv;
            }
          }
        }
      }
#pragma unroll
      for (int s = 0; s < C::kSteps; ++s) {
        if (s + 1 < C::kSteps) {
          read_frags(base + ks, s + 1, (s + 1) & 1);
          mfma_step(s, s & 1, (base + ks) & 1);
          // alternate MFMA and LDS read (the next step's fragments): bursts of
          // reads stall the issuing waves, alternating keeps the matrix pipe fed
          if (kFP8 && (s + 1) % 2 != 0)  // FP8 weights are read every other step
            sched_alternate<MB, MB * NB>();
          else
            sched_alternate<MB + (kFP4 ? 0 : NB), MB * NB>();
        } else {
          const bool more = ks + 1 < nKc;
          __builtin_amdgcn_sched_barrier(0);
          wait_lgkmcnt0();  // this wave's reads of stage ks have returned
          if (more) {
            if (ks + kStages - 1 < nKc)
              wait_vmcnt<(kStages - 2) * C::kLoads>();  // stage ks + 1 landed
            else
              wait_vmcnt<0>();
          }
          stage_barrier();  // stage ks + 1 visible; nobody reads stage ks any more
          if (ks + kStages < nKc) MOE_ISSUE_STAGE(ks + kStages, base + ks + kStages);
          __builtin_amdgcn_sched_barrier(0);
          if (more) read_frags(base + ks + 1, 0, 0);
          mfma_step(s, s & 1, (base + ks) & 1);
          if (more) sched_alternate<MB + (kFP4 ? 2 * NB : NB), MB * NB>();
        }
      }
    }
    if constexpr (kFP8) {
#pragma unroll
      for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int n = 0; n < NB; ++n) acc[m][n] *= rsc[n];
    }

    if (has_next) {
      // The next item's first stages go out before this item's epilogue, so
      // their latency overlaps it.  The wait covers every load issued so far
      // (the next item's inputs among them); the barrier frees all stage
      // buffers (and the other scale buffer).
      wait_vmcnt<0>();
      stage_barrier();
      set_src(xj, x0, xe, n0x, rows_nxt, X.k0);
#pragma unroll
      for (int st = 0; st < kStages; ++st)
        if (st < X.k1 - X.k0) MOE_ISSUE_STAGE(st, base + nKc + st);
    } else {
      wait_vmcnt<0>();  // the gates: nothing else is in flight any more
    }

    // ---- epilogue (store_tile_rows; the router's float32 products below)
    if (kTail && U.u >= 0) {
      // a part of a split tail item: its float32 partial sums, for
      // tail_reduce_kernel (stores only: nothing waits for the next unit's
      // stages here)
      f32x4_t* dst = partial_at<MB, NB>(a.tail + (size_t)U.u * kTailTileFloats, wave, l);
#pragma unroll
      for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int n = 0; n < NB; ++n)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            dst[((m * NB + n) * 4 + r) * kWave] =
                f32x4_t{acc[m][n][4 * r], acc[m][n][4 * r + 1], acc[m][n][4 * r + 2],
                        acc[m][n][4 * r + 3]};
    } else if constexpr (kRouter) {
      // float32 products; 16-byte stores where a run of 16 columns is whole
      // and aligned, else one column at a time (no loads here: a load would
      // wait for the next item's stages already in flight)
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        const int p = c0 + arow_base + m * 32;
        if (p < ce) {
          float* orow =
              a.out_f32 + ((long long)(U.u > 0 ? U.u : 0) * a.rows + p) * a.Nout;  // part plane
#pragma unroll
          for (int n = 0; n < NB; ++n) {
            const int col = n0c + wn * NB * 32 + n * 32 + 16 * g;
            if (col + 16 <= a.Nout && (a.Nout & 3) == 0) {
#pragma unroll
              for (int q = 0; q < 16; q += 4) {
                *reinterpret_cast<f32x4_t*>(orow + col + q) =
                    f32x4_t{acc[m][n][q], acc[m][n][q + 1], acc[m][n][q + 2], acc[m][n][q + 3]};
              }
            } else {
#pragma unroll
              for (int q = 0; q < 16; ++q)
                if (col + q < a.Nout) orow[col + q] = acc[m][n][q];
            }
          }
        }
      }
    } else {
      store_tile_rows<MB, NB, kGateUp>(a, acc, c0, ce, n0c, arow_base, wn, g, gw);
    }

    if (!has_next) break;
    ++kc;
    base += nKc;
    U = X;
    cj = xj, c0 = x0, ce = xe, n0c = n0x;
    xj = yj, x0 = y0, xe = ye, n0x = n0y;
#pragma unroll
    for (int i = 0; i < kRows; ++i) rows_cur[i] = rows_nxt[i];
    parity ^= 1;
  }
#undef MOE_ISSUE_STAGE
}

// Sums of the split tail items (tail_plan): one wave per output block of a
// GEMM wave of a tail item (gate/up: the block and its up block), which adds
// that block's partial sums in part order (a fixed order: the result does
// not depend on which part finished first), with up to four parts' loads in
// flight, and runs the GEMM's epilogue on it.  Launched after the GEMM on the
// same stream, on a small grid whose waves stride over the blocks; does
// nothing when the GEMM split no item.
template <int MB, int WM, int NB, int WN, bool kGateUp>
__global__ __launch_bounds__(256) void tail_reduce_kernel(GemmArgs a, int nK, int align) {
  constexpr int kWaves = WM * WN;
  constexpr int BNW = 32 * NB * WN;
  constexpr int kOut = kGateUp ? NB / 2 : NB;  // output blocks per (GEMM wave, m)
  constexpr int kJobs = kWaves * MB * kOut;    // output blocks per tail item
  constexpr int kB = kGateUp ? 2 : 1;          // partial blocks per output block
  constexpr int kChunk = 4;                    // parts loaded at a time
  const int n_mtiles = *a.ntiles;
  const TailPlan tp = tail_plan(n_mtiles * a.n_tiles_n, a.vw, nK, align);
  if (tp.s <= 1) return;
  const int l = lane_id();
  const int stride = gridDim.x * 4;
  for (int job = blockIdx.x * 4 + (int)threadIdx.x / kWave; job < tp.rem * kJobs;
       job += stride) {
    const int t = job / kJobs, jr = job % kJobs;
    const int w = jr / (MB * kOut), m = (jr / kOut) % MB, n = jr % kOut;
    f32x16_t acc[kB];
    for (int q0 = 0; q0 < tp.s; q0 += kChunk) {
      f32x4_t buf[kChunk][kB][4];
#pragma unroll
      for (int i = 0; i < kChunk; ++i) {
        if (q0 + i < tp.s) {
          // part q of tail item t is unit q * rem + t
          const f32x4_t* src = partial_at<MB, NB>(
              a.tail + (size_t)((q0 + i) * tp.rem + t) * kTailTileFloats, w, l);
#pragma unroll
          for (int b = 0; b < kB; ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              buf[i][b][r] = src[((m * NB + n + b * kOut) * 4 + r) * kWave];
        }
      }
#pragma unroll
      for (int i = 0; i < kChunk; ++i) {
        if (q0 + i < tp.s) {
#pragma unroll
          for (int b = 0; b < kB; ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
              for (int e = 0; e < 4; ++e)
                acc[b][4 * r + e] =
                    q0 + i == 0 ? buf[i][b][r][e] : acc[b][4 * r + e] + buf[i][b][r][e];
        }
      }
    }
    const int2 pl =
        place_item(tp.full + t, a.group_m, n_mtiles, a.n_tiles_n, kGateUp ? BNW / 2 : BNW);
    const int4 tile = a.tiles[pl.x];
    const int p = tile.y + (w % WM) * MB * 32 + (l & 31) + m * 32;
    if (p < tile.z) {
      const float gw = (!kGateUp && a.topk_w) ? a.topk_w[a.sorted_slot[p]] : 1.0f;
      store_block<kGateUp>(a, acc[0], acc[kB - 1], p,
                           pl.y + (w / WM) * kOut * 32 + n * 32 + 16 * (l >> 5), gw);
    }
  }
}

// ---- float32 path: LDS-staged tiles on the fp32 matrix cores
// A tile is 32 token rows of one expert segment x 128 output columns; each of
// the four waves owns a 32 x 32 block (gate/up: a gate and an up block of the
// same 32 features).  Per 32-deep K stage the workgroup stages the tile's
// activation rows (gate/up: gathered through sorted_slot) and weight rows
// into LDS K-major ([k][row], so the 32 lanes that share a K index read 32
// consecutive words: no bank conflicts), then each wave runs 16
// v_mfma_f32_32x32x2_f32 per block (float32 products and sums throughout).
// The float32 problems are small, so a stage's time is the latency of its
// loads: each thread holds the next kF32Ahead stages' loads in registers, and
// the LDS stages alternate between two buffers, one barrier per stage.
constexpr int kF32BM = 32;
constexpr int kF32BN = 128;
constexpr int kF32BK = 32;
constexpr int kF32Ahead = 2;

template <bool kGateUp>
__global__ __launch_bounds__(256) void grouped_f32_kernel(GemmArgs a) {
  constexpr int kMats = kGateUp ? 2 : 1;
  constexpr int kWv = kF32BN / 32;  // weight float4 loads per thread and matrix
  __shared__ float As[2][kF32BK][kF32BM];
  __shared__ float Bs[2][kMats][kF32BK][kF32BN];
  const int n_items = *a.ntiles * a.n_tiles_n;
  const float* A = reinterpret_cast<const float*>(a.A);
  const float* W0 = static_cast<const float*>(a.W0);
  const float* W1 = static_cast<const float*>(a.W1);
  float* out = reinterpret_cast<float*>(a.out);
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int l = lane_id();
  const int nK = a.K / kF32BK;
  // staging: thread tid copies float4 chunk (tid % 8) of K of activation row
  // tid / 8, and of weight rows tid / 8 + 32 i
  const int sr = tid / 8, sk = (tid % 8) * 4;
  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int4 tile = a.tiles[item / a.n_tiles_n];
    const int j = tile.x, row0 = tile.y, row_end = tile.z;
    const int n0 = (item % a.n_tiles_n) * kF32BN;
    const int p_st = min(row0 + sr, row_end - 1);
    const long long arow = kGateUp ? (long long)(a.sorted_slot[p_st] / a.k) : (long long)p_st;
    const float* asrc = A + arow * a.K + sk;
    const float* wsrc[kMats][kWv];
#pragma unroll
    for (int m = 0; m < kMats; ++m)
#pragma unroll
      for (int i = 0; i < kWv; ++i)
        wsrc[m][i] = (m == 0 ? W0 : W1) +
                     ((long long)j * a.Nout + min(n0 + sr + 32 * i, a.Nout - 1)) * a.K + sk;
    // the loads of stage s sit in register set s % 2, which is also its LDS
    // buffer (register and LDS buffers indexed by compile-time constants)
    static_assert(kF32Ahead == 2, "two register sets, two LDS buffers");
    f32x4_t ra[2];
    f32x4_t rw[2][kMats][kWv];
    auto load = [&](int s, auto bc) {
      constexpr int b = decltype(bc)::value;
      ra[b] = *reinterpret_cast<const f32x4_t*>(asrc + s * kF32BK);
#pragma unroll
      for (int m = 0; m < kMats; ++m)
#pragma unroll
        for (int i = 0; i < kWv; ++i)
          rw[b][m][i] = *reinterpret_cast<const f32x4_t*>(wsrc[m][i] + s * kF32BK);
    };
    f32x16_t acc[kMats];
#pragma unroll
    for (int m = 0; m < kMats; ++m) acc[m] = f32x16_t{};
    // stage s: into LDS buffer s % 2 (its last readers, the MFMAs of stage
    // s - 2, are behind the barrier of stage s - 1), barrier, the loads of
    // stage s + 2 into the freed registers, then the MFMAs
    auto stage = [&](int s, auto bc) {
      constexpr int b = decltype(bc)::value;
#pragma unroll
      for (int q = 0; q < 4; ++q) As[b][sk + q][sr] = ra[b][q];
#pragma unroll
      for (int m = 0; m < kMats; ++m)
#pragma unroll
        for (int i = 0; i < kWv; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) Bs[b][m][sk + q][sr + 32 * i] = rw[b][m][i][q];
      __syncthreads();
      if (s + 2 < nK) load(s + 2, bc);
      // v_mfma_f32_32x32x2_f32: lane l gives A[row l % 32][k l / 32] and
      // B[k l / 32][column l % 32]
#pragma unroll
      for (int kk = 0; kk < kF32BK; kk += 2) {
        const float av2 = As[b][kk + l / 32][l % 32];
#pragma unroll
        for (int m = 0; m < kMats; ++m)
          acc[m] = __builtin_amdgcn_mfma_f32_32x32x2f32(
              av2, Bs[b][m][kk + l / 32][wave * 32 + l % 32], acc[m], 0, 0, 0);
      }
    };
    constexpr std::integral_constant<int, 0> kB0{};
    constexpr std::integral_constant<int, 1> kB1{};
    load(0, kB0);
    if (nK > 1) load(1, kB1);
    for (int s = 0; s < nK; s += 2) {
      stage(s, kB0);
      if (s + 1 < nK) stage(s + 1, kB1);
    }
    // the next item's first stage goes to LDS buffer 0, last read by this
    // item's stage nK - 2
    __syncthreads();
    // result block [token row][column]: lane l holds column l % 32, register
    // r row 8 (r / 4) + 4 (l / 32) + r % 4
    const int col = n0 + wave * 32 + l % 32;
    if (col < a.Nout) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int p = row0 + 8 * (r / 4) + 4 * (l / 32) + (r % 4);
        if (p < row_end) {
          float v;
          if constexpr (kGateUp) {
            const float gs = acc[0][r];
            v = gs / (1.0f + expf(-gs)) * acc[kMats - 1][r];
          } else {
            v = acc[0][r] * (a.topk_w ? a.topk_w[a.sorted_slot[p]] : 1.0f);
          }
          out[(long long)p * a.Nout + col] = v;
        }
      }
    }
  }
}

// ---- decode-sized GEMMs: weights streamed by each wave into registers
// With a handful of rows per expert the GEMMs only stream weights from HBM.
// Here every wave works on its own: an item is (M tile of at most 32 rows of
// one expert, NB weight blocks of 32 rows; gate/up: NB/2 gate blocks and the
// up blocks of the same features), and the wave loads its blocks' weights
// straight into registers kD slices ahead of its MFMAs, the tile's
// activation rows (L2 hits: a decode batch is small) in the same stream.  No
// LDS and no barrier: nothing holds a wave's loads back but its own register
// ring, and the next item's first slices are in flight while the current
// item finishes.  A slice is 16 K values (bf16: one MFMA step) or 64 (MXFP4:
// per lane and block one 16-byte chunk of 32 codes and its E8M0 scale, four
// MFMA steps).  K order, operand layout and epilogue are the staged kernel's
// (weights as the A operand in the permuted row order, so a lane's 16 result
// registers are 16 consecutive features of one row), so both give the same
// bits.  Either weight layout: a lane's offsets inside a 64-K unit of a block
// are per-lane constants, everything else is a scalar added at issue.
template <bool kGateUp, int kWBits, int NB, int kD>
struct StreamCfg {
  static constexpr bool kFP4 = kWBits == 4;
  static constexpr int kSliceK = kFP4 ? 64 : 16;   // K values per slice
  static constexpr int kTok = kSliceK / 16;        // 16-byte activation loads per slice
  static constexpr int kLoads = NB * (kFP4 ? 2 : 1) + kTok;  // vector memory ops per slice
  static constexpr int kRowB = 64 * kWBits / 8;    // bytes of one weight row in a 64-K unit
  static_assert(kWBits == 16 || kFP4, "bf16 or MXFP4 weights");
  static_assert(!kGateUp || NB % 2 == 0, "gate/up pairs gate and up blocks");
  static_assert(kD >= 2 && (kD - 1) * kLoads < 64, "vmcnt budget");
  static_assert(kFP4 || kD % 4 == 0, "bf16: whole 64-K units per turn of the ring");
};

constexpr int kStreamWaves = 4;

// f(integral_constant<int, I>) for I = B .. E - 1, unrolled at compile time
// (ring entries and wait counts must be constants)
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

template <bool kGateUp, int kWBits, int NB, int kD, int kMinBlocks>
__global__ __launch_bounds__(kWave* kStreamWaves, kMinBlocks) void stream_gemm_kernel(GemmArgs a) {
  using C = StreamCfg<kGateUp, kWBits, NB, kD>;
  constexpr bool kFP4 = C::kFP4;
  constexpr int H = kGateUp ? NB / 2 : NB;  // output blocks of an item
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int l = lane_id();
  const int g = l >> 5;   // which 8 of an MFMA step's 16 K values this lane holds
  const int r = l & 31;   // MFMA row (weights) and column (tokens) of this lane
  const int nsplit = a.ksplit;      // K ranges per (M tile, N group)
  const int nS = a.K / C::kSliceK / nsplit;  // slices per item, a multiple of kD (host)
  const int ntn = a.n_tiles_n;      // N groups per M tile
  const int n_items = *a.ntiles * ntn * nsplit;
  const int stride = gridDim.x * kStreamWaves;
  // item pairs (2p, 2p + 1: neighbouring N groups of one M tile, which share
  // activation rows and the 128-byte lines of their scales) round-robin over
  // the workgroups first, so that every CU gets the same number of busy
  // waves; the two items of a pair run on two waves of one workgroup
  // (measured: MXFP4 gate/up 3 % faster than single items round-robin)
  int it = 2 * (blockIdx.x + gridDim.x * (wave >> 1)) + (wave & 1);
  if (it >= n_items) return;

  // per-lane constants: row r of a weight block holds feature fr (the
  // staged kernel's permuted order); offsets inside a 64-K unit
  const int fr = (r & ~31) | (((r >> 2) & 1) << 4) | (((r >> 3) & 3) << 2) | (r & 3);
  const uint32_t row_bytes = (uint32_t)a.K * kWBits / 8;  // one full weight row
  const uint32_t unit_step = a.blocked ? 32u * C::kRowB : (uint32_t)C::kRowB;  // per 64 K
  const uint32_t wmat = (uint32_t)a.Nout * row_bytes;
  // (blocked: chunk q of the unit's rows is the 1 KB operand load q, lane l
  // at 16 l; row-major: row fr, K chunk 2 q + g)
  uint32_t voffW[kFP4 ? 1 : 4];
  if constexpr (kFP4) {
    voffW[0] = a.blocked ? 16u * l : (uint32_t)fr * row_bytes + 16u * g;
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      voffW[q] = a.blocked ? 1024u * q + 16u * l : (uint32_t)fr * row_bytes + 16u * (2 * q + g);
  }

  // per-item state
  __amdgpu_buffer_rsrc_t rsA, rsW0, rsW1, rsS0, rsS1;
  uint32_t voffA = 0, voffS = 0;
  uint32_t sW[NB];  // byte offset of block n's rows in its matrix
  uint32_t sS[NB];  // MXFP4: first feature of block n
  int sbase = 0;    // first slice of the item's K range (a multiple of kD)
  auto setup = [&](int item, int4 t, int ss) {
    const int grp = (item / nsplit) % ntn;
    sbase = (item % nsplit) * nS;
    const int j = __builtin_amdgcn_readfirstlane(t.x);
    const int p = min(__builtin_amdgcn_readfirstlane(t.y) + r, __builtin_amdgcn_readfirstlane(t.z) - 1);
    const uint32_t arow = kGateUp ? (uint32_t)(ss / a.k) : (uint32_t)p;
    rsA = buffer_rsrc(a.A, a.a_bytes);
    voffA = arow * (uint32_t)a.K * 2u + (kFP4 ? 64u : 16u) * g;
    rsW0 = buffer_rsrc(static_cast<const unsigned char*>(a.W0) + (size_t)j * wmat, wmat);
    rsW1 = kGateUp ? buffer_rsrc(static_cast<const unsigned char*>(a.W1) + (size_t)j * wmat, wmat)
                   : rsW0;
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      const int fb = min(grp * H + (n % H), a.Nout / 32 - 1);
      sW[n] = (uint32_t)fb * 32u * row_bytes;
      sS[n] = (uint32_t)fb * 32u;
    }
    if constexpr (kFP4) {
      const uint32_t smat = (uint32_t)(a.K / 32) * a.Nout;
      rsS0 = buffer_rsrc(static_cast<const unsigned char*>(a.S0) + (size_t)j * smat, smat);
      rsS1 = kGateUp ? buffer_rsrc(static_cast<const unsigned char*>(a.S1) + (size_t)j * smat, smat)
                     : rsS0;
      voffS = (uint32_t)g * a.Nout + fr;
    }
  };

  // register ring
  u32x4_t wb[kD][NB];
  u32x4_t tb[kD][C::kTok];
  uint32_t sb[kD][kFP4 ? NB : 1];
  // slice s of the item set up last into ring entry e (e = s mod kD)
  auto issue = [&](int s, int e) {
    s += sbase;
    if constexpr (kFP4) {
#pragma unroll
      for (int n = 0; n < NB; ++n) {
        wb[e][n] = __builtin_amdgcn_raw_buffer_load_b128(kGateUp && n >= H ? rsW1 : rsW0, voffW[0],
                                                         sW[n] + (uint32_t)s * unit_step, 2);
        sb[e][n] = __builtin_amdgcn_raw_buffer_load_b8(kGateUp && n >= H ? rsS1 : rsS0, voffS,
                                                       sS[n] + (uint32_t)(2 * s) * a.Nout, 0);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q)
        tb[e][q] = __builtin_amdgcn_raw_buffer_load_b128(rsA, voffA + 16u * q, (uint32_t)s * 128u, 0);
    } else {
      const int q = e & 3;  // step inside the 64-K unit (kD % 4 == 0, s = e mod 4)
#pragma unroll
      for (int n = 0; n < NB; ++n)
        wb[e][n] = __builtin_amdgcn_raw_buffer_load_b128(kGateUp && n >= H ? rsW1 : rsW0, voffW[q],
                                                         sW[n] + (uint32_t)(s >> 2) * unit_step, 2);
      tb[e][0] = __builtin_amdgcn_raw_buffer_load_b128(rsA, voffA, (uint32_t)s * 32u, 0);
    }
  };
  f32x16_t acc[NB];
  auto compute = [&](int e) {
    if constexpr (kFP4) {
      float sc[NB];
#pragma unroll
      for (int n = 0; n < NB; ++n) sc[n] = e8m0_to_f32(sb[e][n]);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bf16x8_t tok = __builtin_bit_cast(bf16x8_t, tb[e][q]);
#pragma unroll
        for (int n = 0; n < NB; ++n)
          acc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(e2m1x8_to_bf16x8(wb[e][n][q], sc[n]), tok,
                                                           acc[n], 0, 0, 0);
      }
    } else {
      const bf16x8_t tok = __builtin_bit_cast(bf16x8_t, tb[e][0]);
#pragma unroll
      for (int n = 0; n < NB; ++n)
        acc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, wb[e][n]), tok,
                                                         acc[n], 0, 0, 0);
    }
  };

  // Item metadata runs ahead of the item: the tile of the item after next
  // and the gather slot of the next item are loaded one item before they
  // are used, so that no address computation waits on a load (a wait right
  // behind a load would drain every slice in flight).
  // (an index the compiler cannot prove wave-uniform keeps a loaded tile in
  // vector registers until setup reads it: moving it to scalar registers
  // right at the load would wait for it there)
  auto tile_of = [&](int item) -> int4 {
    int opaque_zero;
    asm volatile("v_mov_b32 %0, 0" : "=v"(opaque_zero));
    return item < n_items ? a.tiles[item / nsplit / ntn + opaque_zero] : make_int4(0, 0, 1, 0);
  };
  auto slot_of = [&](int4 t) -> int { return a.sorted_slot[min(t.y + r, t.z - 1)]; };
  int4 tc = tile_of(it);
  int4 tn = tile_of(it + stride);
  int4 tnn = tile_of(it + 2 * stride);
  int ss_c = slot_of(tc);
  int ss_n = slot_of(tn);
  float gate = (!kGateUp && a.topk_w) ? a.topk_w[ss_c] : 1.0f;
  setup(it, tc, ss_c);
  // (sched_barrier keeps every ring step in slice order, in the prologue as
  // in the loops: the compiler's own vmcnt waits then match the explicit
  // ones instead of assuming the worst order)
  static_for<0, kD>([&](auto e) {
    issue(e, e);
    __builtin_amdgcn_sched_barrier(0);
  });

  for (;;) {
    const int itn = it + stride;
    const bool has_next = itn < n_items;
#pragma unroll
    for (int n = 0; n < NB; ++n) acc[n] = f32x16_t{};
    for (int s0 = 0; s0 < nS - kD; s0 += kD) {
      static_for<0, kD>([&](auto e) {
        wait_vmcnt<(kD - 1) * C::kLoads>();
        compute(e);
        issue(s0 + kD + e, e);
        __builtin_amdgcn_sched_barrier(0);
      });
    }
    // last turn of the ring: the next item's first slices take the freed
    // entries (the wait counts stay those of the steady loop)
    const int grp_c = (it / nsplit) % ntn, sp_c = it % nsplit;
    const int row0 = __builtin_amdgcn_readfirstlane(tc.y), rend = __builtin_amdgcn_readfirstlane(tc.z);
    const float gate_c = gate;
    int ss_nn = 0;
    int4 tnnn = make_int4(0, 0, 1, 0);
    if (has_next) {
      ss_nn = slot_of(tnn);
      tnnn = tile_of(itn + 2 * stride);
      gate = (!kGateUp && a.topk_w) ? a.topk_w[ss_n] : 1.0f;
      setup(itn, tn, ss_n);
      static_for<0, kD>([&](auto e) {
        wait_vmcnt<(kD - 1) * C::kLoads>();
        compute(e);
        issue(e, e);
        __builtin_amdgcn_sched_barrier(0);
      });
    } else {
      // nothing issued behind: wait for exactly the slices still ahead
      static_for<0, kD>([&](auto e) {
        wait_vmcnt<(kD - 1 - decltype(e)::value) * C::kLoads>();
        compute(e);
      });
    }

    // epilogue: register q of block n is feature 16 g + q of the block
    const int p = row0 + r;
    if (nsplit > 1) {
      // float32 partial products of this K range (gate/up: gate, then up columns)
      if (p < rend) {
        float* prow = a.part + ((long long)sp_c * a.part_rows + p) * (kGateUp ? 2 * a.Nout : a.Nout);
#pragma unroll
        for (int n = 0; n < NB; ++n) {
          const int col = (kGateUp && n >= H ? a.Nout : 0) + grp_c * H * 32 + (n % H) * 32 + 16 * g;
#pragma unroll
          for (int q = 0; q < 16; q += 4)
            *reinterpret_cast<f32x4_t*>(prow + col + q) =
                f32x4_t{acc[n][q], acc[n][q + 1], acc[n][q + 2], acc[n][q + 3]};
        }
      }
    } else if (p < rend) {
      uint16_t* orow = a.out + (long long)p * a.Nout;
#pragma unroll
      for (int n = 0; n < H; ++n) {
        const int col = grp_c * H * 32 + n * 32 + 16 * g;
        if (col < a.Nout) {
          float h[16];
#pragma unroll
          for (int q = 0; q < 16; ++q)
            h[q] = kGateUp ? silu_f32(acc[n][q]) * acc[n + (kGateUp ? H : 0)][q] : acc[n][q] * gate_c;
          *reinterpret_cast<u32x4_t*>(orow + col) =
              u32x4_t{pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]), pack_bf16x2(h[4], h[5]),
                      pack_bf16x2(h[6], h[7])};
          *reinterpret_cast<u32x4_t*>(orow + col + 8) =
              u32x4_t{pack_bf16x2(h[8], h[9]), pack_bf16x2(h[10], h[11]),
                      pack_bf16x2(h[12], h[13]), pack_bf16x2(h[14], h[15])};
        }
      }
    }
    if (!has_next) break;
    it = itn;
    tc = tn;
    tn = tnn;
    tnn = tnnn;
    ss_n = ss_nn;
  }
}

// Sum of the K-range partial products in split order, then the epilogue of
// the unsplit GEMM: gate/up h = silu(gate) * up, down y = sum * gate(row).
// Thread per 8 output columns of a kept row (rows past offsets[El] are not
// written: no tile covers them).
template <bool kGateUp>
__global__ __launch_bounds__(256) void split_reduce_kernel(GemmArgs a, int El) {
  const int n8 = a.Nout / 8;
  const long long o = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const int p = (int)(o / n8);
  const int c = (int)(o % n8) * 8;
  if (p >= a.offsets[El]) return;
  const int w = kGateUp ? 2 * a.Nout : a.Nout;
  float v[8], u[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) v[q] = u[q] = 0.f;
  for (int sp = 0; sp < a.ksplit; ++sp) {
    const float* prow = a.part + ((long long)sp * a.part_rows + p) * w;
    const f32x4_t g0 = *reinterpret_cast<const f32x4_t*>(prow + c);
    const f32x4_t g1 = *reinterpret_cast<const f32x4_t*>(prow + c + 4);
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] += g0[q], v[q + 4] += g1[q];
    if constexpr (kGateUp) {
      const f32x4_t u0 = *reinterpret_cast<const f32x4_t*>(prow + a.Nout + c);
      const f32x4_t u1 = *reinterpret_cast<const f32x4_t*>(prow + a.Nout + c + 4);
#pragma unroll
      for (int q = 0; q < 4; ++q) u[q] += u0[q], u[q + 4] += u1[q];
    }
  }
  float h[8];
  const float gate = (!kGateUp && a.topk_w) ? a.topk_w[a.sorted_slot[p]] : 1.0f;
#pragma unroll
  for (int q = 0; q < 8; ++q) h[q] = kGateUp ? silu_f32(v[q]) * u[q] : v[q] * gate;
  *reinterpret_cast<u32x4_t*>(a.out + (long long)p * a.Nout + c) =
      u32x4_t{pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]), pack_bf16x2(h[4], h[5]),
              pack_bf16x2(h[6], h[7])};
}

// ---- launch plumbing
// What a launch needs to know about the device and the caller's grid cap,
// read once per library call (nothing is cached between calls).
struct LaunchEnv {
  int num_cu;          // compute units of the current device
  long long max_wg;    // MOE_MI355X_MAX_WORKGROUPS, or 0 (no cap)
};

// MOE_MI355X_MAX_WORKGROUPS caps the persistent GEMM grid (rounded up to a
// multiple of 8).  Results do not depend on it: every output element comes
// from one tile with a fixed K order.  Tests use it to give each workgroup
// many items.
LaunchEnv launch_env() {
  LaunchEnv env{256, 0};
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) == hipSuccess &&
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
    env.num_cu = n;
  if (const char* v = getenv("MOE_MI355X_MAX_WORKGROUPS")) env.max_wg = atoll(v);
  return env;
}

template <int MB, int WM, int NB, int WN, bool kGateUp, int kWBits, int kBK, int kStages,
          int kMinBlocks, bool kRouter, bool kBlk>
hipError_t launch_gemm_l(const GemmArgs& a, long long max_items, const LaunchEnv& env,
                         hipStream_t st) {
  using C = Cfg<MB, WM, NB, WN, kGateUp, kWBits, kBK, kStages>;
  auto kern =
      grouped_gemm_kernel<MB, WM, NB, WN, kGateUp, kWBits, kBK, kStages, kMinBlocks, kRouter, kBlk>;
  static std::atomic<uint64_t> attr_done{0};  // per instantiation: devices already set
  hipError_t e = set_lds_attr(reinterpret_cast<const void*>(kern), C::kLds, attr_done);
  if (e != hipSuccess) return e;
  long long grid = (long long)env.num_cu * kMinBlocks;
  const long long need = (max_items + kNumXcd - 1) / kNumXcd * kNumXcd;
  if (need < grid) grid = need;
  if (env.max_wg > 0 && env.max_wg < grid) grid = env.max_wg;
  grid = (grid + kNumXcd - 1) / kNumXcd * kNumXcd;
  if (grid < kNumXcd) grid = kNumXcd;
  // stages, then the FP8 scales of two items
  const size_t lds = (size_t)kStages * C::kStage + (C::kFP8 ? 2u * C::kScaleSets * (a.K / 128) * 4 : 0);
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(C::kThreads), lds, st, a);
  return hipGetLastError();
}

// the kernel for the weight layout in a.blocked (blocked units are 64 K deep:
// plans with other K steps take row-major weights only)
template <int MB, int WM, int NB, int WN, bool kGateUp, int kWBits, int kBK, int kStages,
          int kMinBlocks, bool kRouter = false>
hipError_t launch_gemm(const GemmArgs& a, long long max_items, const LaunchEnv& env,
                       hipStream_t st) {
  if constexpr (kBK == 64 && !kRouter) {
    if (a.blocked)
      return launch_gemm_l<MB, WM, NB, WN, kGateUp, kWBits, kBK, kStages, kMinBlocks, kRouter,
                           true>(a, max_items, env, st);
  } else {
    if (a.blocked) return hipErrorInvalidValue;
  }
  return launch_gemm_l<MB, WM, NB, WN, kGateUp, kWBits, kBK, kStages, kMinBlocks, kRouter, false>(
      a, max_items, env, st);
}

// A prefill-sized GEMM with the tail split (a.vw virtual workers), then the
// sums of its split tail items.  The grid covers all virtual workers, as the
// tail parts can outnumber the items.
template <int MB, int WM, int NB, int WN, bool kGateUp, int kWBits, int kBK, int kStages,
          int kMinBlocks>
hipError_t launch_prefill(const GemmArgs& a, long long max_items, const LaunchEnv& env,
                          hipStream_t st) {
  hipError_t e = launch_gemm<MB, WM, NB, WN, kGateUp, kWBits, kBK, kStages, kMinBlocks>(
      a, std::max<long long>(max_items, a.vw), env, st);
  // (no item can be split when K holds fewer than two parts' worth of stages)
  if (e != hipSuccess || a.vw < kNumXcd || a.K / kBK < 2 * kMinPartStages) return e;
  // then the sums of the split tail items: 512 workgroups of 4 waves stride
  // over the output blocks (Mixtral's down GEMM: 4096 blocks, 31 us on 64
  // workgroups)
  hipLaunchKernelGGL((tail_reduce_kernel<MB, WM, NB, WN, kGateUp>), dim3(512), dim3(256), 0, st,
                     a, a.K / kBK, kWBits == 8 ? 128 / kBK : 1);
  return hipGetLastError();
}

// Wave-streamed decode GEMMs: one item per wave, item pairs spread over
// kMinBlocks workgroups per CU (never more workgroups than pairs).
template <bool kGateUp, int kWBits, int NB, int kD, int kMinBlocks>
hipError_t launch_stream(const GemmArgs& a, long long max_items, const LaunchEnv& env,
                         hipStream_t st) {
  using C = StreamCfg<kGateUp, kWBits, NB, kD>;
  // whole turns of the ring per item (and K range), whole items per output row
  if (a.ksplit < 1 || (a.K / C::kSliceK) % (kD * a.ksplit) != 0 ||
      a.Nout % (32 * (kGateUp ? NB / 2 : NB)) != 0 || (a.ksplit > 1 && a.part == nullptr))
    return hipErrorInvalidValue;
  long long grid = (long long)env.num_cu * kMinBlocks;
  if ((max_items + 1) / 2 < grid) grid = (max_items + 1) / 2;
  if (env.max_wg > 0 && env.max_wg < grid) grid = env.max_wg;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL((stream_gemm_kernel<kGateUp, kWBits, NB, kD, kMinBlocks>),
                     dim3((unsigned)grid), dim3(kWave * kStreamWaves), 0, st, a);
  return hipGetLastError();
}

// Tile plans.  Decode (a handful of rows per expert): 32 x 256 tiles, four
// waves side by side along N, 64-deep K steps, 4 stages; from 17 to 64 rows
// per expert on average (bf16), 64 x 256 tiles, so that an expert's weights
// are streamed by one M tile instead of two or three.  bf16 prefill: eight
// waves of 64 x 128, 64-deep K steps and 2 stages, as 128 x 512 tiles when
// experts hold a few hundred rows (less M padding) or 256 x 256 from 512 rows
// per expert on average (fewer bytes staged per MFMA: the tile's loads come
// through each compute unit's L1 at a rate set by the L1's misses in flight
// and their latency, so bytes per MFMA decide; the Qwen3 prefill, 512 rows per
// expert, runs 4 % faster on 256 x 256 than on 128 x 512 despite 15 % M
// padding against 12 %).  (64-deep steps read whole
// 128-byte lines of every row per stage and halve the barriers: 9-14 % faster
// than 32-deep steps with 4 stages.)  FP8 weights: 128 x 512 tiles of eight
// waves side by side along N (128 x 64 each, so that each weight block is
// widened by one wave), 64-deep K steps (one byte per code) and 2 stages
// (7 % faster than a 2 x 4 wave grid with 3 stages).  MXFP4 weights: at
// decode sizes, on blocked weights, the wave-streamed GEMMs (measured on the Qwen3 decode step,
// gate/up 49.2 -> 42.8 us and down 28.7 -> 25.7 us against the staged 32 x 256
// tile with three workgroups per CU: a staged MXFP4 block is a quarter of a
// bf16 one, so the per-stage wait and barrier dominated); else the FP8
// prefill tile shape with 4 stages (0.63 -> 0.42 ms against the 2 x 4 wave
// grid on the Qwen3 prefill).  bf16 decode stays staged: streamed bf16 blocks
// (2 or 4 per wave, 4 to 8 slices ahead, 8 or 12 waves per CU) took
// 137-142 us for the Qwen3 gate/up against 138-140 staged on the same box,
// and their down GEMM 73-75 us against 72-74.
enum class Plan { kF32, kDecode, kDecode64, kWide, kBig, kFp8, kDecodeFp4, kFp4 };

Plan plan_of(const Shape& s) {
  if (s.weight == kF32) return Plan::kF32;
  if (s.weight == kFP4) return s.S <= 64LL * s.El ? Plan::kDecodeFp4 : Plan::kFp4;
  if (s.S <= 16LL * s.El) return Plan::kDecode;
  // bf16: 64-row tiles below 64 slots per expert on average; from 64 on,
  // about half the experts overflow one 64-row tile and would stream their
  // weights twice (Qwen3 shape, T = 1024: 0.349 ms against 0.310 on 128-row
  // tiles; at T = 896, 0.282 against 0.307)
  if (s.weight == kFP8 && s.S <= 64LL * s.El) return Plan::kDecode;
  if (s.S < 64LL * s.El) return Plan::kDecode64;
  if (s.weight == kFP8) return Plan::kFp8;
  return s.S >= 512LL * s.El ? Plan::kBig : Plan::kWide;
}

// prefill-sized tiles (128 or 256 rows): items dealt to virtual workers with
// the tail split
bool uses_tail_split(const Shape& s) {
  const Plan p = plan_of(s);
  return p == Plan::kWide || p == Plan::kBig || p == Plan::kFp8 || p == Plan::kFp4;
}

bool use_decode_tiles(const Shape& s) {
  const Plan p = plan_of(s);
  return p == Plan::kDecode || p == Plan::kDecode64 || p == Plan::kDecodeFp4;
}

int tile_bm(const Shape& s) {
  switch (plan_of(s)) {
    case Plan::kF32: return kF32BM;
    case Plan::kDecode: return 32;
    case Plan::kDecodeFp4: return 32;
    case Plan::kDecode64: return 64;
    case Plan::kBig: return 256;
    default: return 128;
  }
}

size_t max_tiles(const Shape& s, int bm) { return (size_t)((s.S + bm - 1) / bm) + s.El; }

// bf16 decode with very few slots (a handful of touched experts): the
// wave-streamed gate/up GEMM with each item's K range split in ks parts, so
// that the items (at most min(E_l, S) touched experts x groups x ks) about
// fill the 2048 waves of two 4-wave workgroups per CU; 1 (no split: the
// staged plan) when the unsplit items already fill them.  A function of the
// shape only, so the workspace size is too.  (Measured on the Qwen3 shape:
// gate/up 25.9 -> 18.3 us at T = 1, 28.9 -> 24.0 at T = 2, equal at T = 4;
// the down GEMM split the same way was slower from T = 2 on, so it stays
// staged.)
int small_batch_split(const Shape& s, int K, int groups) {
  if (s.weight != kBF16 || plan_of(s) != Plan::kDecode) return 1;
  constexpr long long kWaveSlots = 2048;
  const long long items = std::min<long long>(s.El, s.S) * groups;
  int best = 1;
  for (int ks = 2; ks <= 16; ++ks) {
    if (items * ks > kWaveSlots) break;
    if ((K / 16) % (8 * ks) == 0) best = ks;  // whole turns of the 8-slice ring
  }
  return best;
}

// bytes of the gate/up GEMM's split partial products
size_t split_part_bytes(const Shape& s) {
  const size_t gu = (size_t)small_batch_split(s, s.d, s.F / 32);
  return gu > 1 ? gu * s.S * 2 * s.F * sizeof(float) : 0;
}

}  // namespace

bool use_router_gemm(const Shape& s) { return s.act == kBF16 && s.T >= 1024; }

namespace {
// Router GEMM tiles: 256 x 256 from kRouterBigFrom tokens (bytes staged per
// MFMA as in the prefill expert GEMMs), else 32 x 256 (four waves side by
// side along the experts).  With fewer items than compute units, each tile's
// K range is cut into parts (at least 8 K stages each) so that about one
// item runs per compute unit.
constexpr int kRouterBigFrom = 8192;
struct RouterGemmPlan {
  int bm, ks;
};
RouterGemmPlan router_gemm_plan(const Shape& s) {
  const int bm = s.T >= kRouterBigFrom ? 256 : 32;
  const long long items = (long long)((s.T + bm - 1) / bm) * ((s.E + 255) / 256);
  const int max_ks = std::max(1, std::min(16, s.d / 64 / 8));
  int ks = (int)std::max<long long>(1, std::min<long long>(max_ks, 256 / std::max(items, 1LL)));
  return {bm, ks};
}
}  // namespace

int router_gemm_splits(const Shape& s) { return router_gemm_plan(s).ks; }

hipError_t router_gemm(const Shape& s, const void* x, const void* w_router_t, float* prod,
                       hipStream_t st) {
  const LaunchEnv env = launch_env();
  const RouterGemmPlan rp = router_gemm_plan(s);
  GemmArgs a{};
  a.A = static_cast<const uint16_t*>(x);
  a.a_bytes = (uint32_t)((size_t)s.T * s.d * 2);
  a.k = 1;
  a.W0 = w_router_t;
  a.out_f32 = prod;  // [ks][T][E]
  a.rows = s.T;
  a.K = s.d;
  a.Nout = s.E;
  a.n_tiles_n = (s.E + 255) / 256;
  a.group_m = 1;
  a.ksplit = rp.ks;
  const long long items = (long long)((s.T + rp.bm - 1) / rp.bm) * a.n_tiles_n * rp.ks;
  if (rp.bm == 256)
    return launch_gemm<2, 4, 4, 2, false, 16, 64, 2, 1, true>(a, items, env, st);
  return launch_gemm<1, 1, 2, 4, false, 16, 64, 4, 1, true>(a, items, env, st);
}

FfnSchedule ffn_schedule_view(const Shape& s, void* ws) {
  unsigned char* p = static_cast<unsigned char*>(ws);
  FfnSchedule v;
  v.tiles = reinterpret_cast<int4*>(p);
  v.ntiles = reinterpret_cast<int*>(p + align_up(max_tiles(s, 32) * sizeof(int4)));
  v.bm = tile_bm(s);
  return v;
}

// bytes of the tail split's partial sums (at most kMaxVW tail units of one tile)
size_t tail_part_bytes(const Shape& s) {
  return uses_tail_split(s) ? (size_t)kMaxVW * kTailTileFloats * sizeof(float) : 0;
}

size_t ffn_ws_bytes(const Shape& s) {
  // schedule (at the smallest tile) + tile count + h [S][F] + split partials
  // + tail partials
  return align_up(max_tiles(s, 32) * sizeof(int4)) + align_up(sizeof(int)) +
         align_up((size_t)s.S * s.F * act_bytes(s)) + align_up(split_part_bytes(s)) +
         align_up(tail_part_bytes(s));
}

hipError_t expert_ffn(const Shape& s, const void* x, const int32_t* sorted_slot,
                      const int32_t* offsets, const void* w_gate, const void* w_up,
                      const void* w_down, const void* s_gate, const void* s_up,
                      const void* s_down, const float* topk_w, void* y, void* ws,
                      hipStream_t st, bool schedule_ready, hipEvent_t const* ev) {
  if (s.S == 0) return hipSuccess;
  const LaunchEnv env = launch_env();
  const FfnSchedule sv = ffn_schedule_view(s, ws);
  int4* tiles = sv.tiles;
  int* ntiles = sv.ntiles;
  uint16_t* h = reinterpret_cast<uint16_t*>(static_cast<unsigned char*>(ws) +
                                            align_up(max_tiles(s, 32) * sizeof(int4)) +
                                            align_up(sizeof(int)));
  float* part = reinterpret_cast<float*>(reinterpret_cast<unsigned char*>(h) +
                                         align_up((size_t)s.S * s.F * act_bytes(s)));
  float* tail = reinterpret_cast<float*>(reinterpret_cast<unsigned char*>(part) +
                                         align_up(split_part_bytes(s)));
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
  gu.a_bytes = (uint32_t)((size_t)s.T * s.d * act_bytes(s));
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
  gu.ksplit = 1;
  gu.part = part;
  gu.part_rows = (int)s.S;
  // virtual workers of the tail split: the device's compute units (whole
  // XCDs), so the cut, and the results, depend on the device only
  gu.vw = uses_tail_split(s) && env.num_cu >= kNumXcd
              ? std::min(env.num_cu / kNumXcd * kNumXcd, kMaxVW)
              : 0;
  gu.tail = tail;

  GemmArgs dn = gu;
  dn.A = h;
  // h as one buffer (the wave-streamed decode GEMMs; the staged kernel reads
  // h through per-tile resources)
  dn.a_bytes = (uint32_t)std::min<long long>((long long)s.S * s.F * act_bytes(s), 0xFFFFFFFFLL);
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
  gu.blocked = dn.blocked = s.blocked;
  if (s.weight == kF32) {
    gu.n_tiles_n = (s.F + kF32BN - 1) / kF32BN;
    dn.n_tiles_n = (s.d + kF32BN - 1) / kF32BN;
    // a workgroup per possible item, at most four per CU (the items loop)
    auto grid = [&](int ntn) {
      return (unsigned)std::max<long long>(1, std::min<long long>(4LL * env.num_cu, mt * ntn));
    };
    hipLaunchKernelGGL(grouped_f32_kernel<true>, dim3(grid(gu.n_tiles_n)), dim3(256), 0, st, gu);
    e = hipGetLastError();
    if (e == hipSuccess && ev) e = hipEventRecord(ev[1], st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(grouped_f32_kernel<false>, dim3(grid(dn.n_tiles_n)), dim3(256), 0, st, dn);
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
        e = launch_gemm<1, 1, 2, 4, true, 8, 64, 4, 2>(gu, mt * gu.n_tiles_n, env, st);
        if (e == hipSuccess && ev) e = hipEventRecord(ev[1], st);
        if (e == hipSuccess) e = launch_gemm<1, 1, 2, 4, false, 8, 64, 4, 2>(dn, mt * dn.n_tiles_n, env, st);
      } else {
        // very few slots: the gate/up GEMM wave-streamed with split K ranges,
        // then the sums and SiLU
        const int ks_gu = small_batch_split(s, s.d, s.F / 32);
        if (ks_gu > 1) {
          gu.n_tiles_n = s.F / 32;
          gu.ksplit = ks_gu;
          e = launch_stream<true, 16, 2, 8, 2>(gu, mt * gu.n_tiles_n * ks_gu, env, st);
          if (e == hipSuccess) {
            const long long n = s.S * (s.F / 8);
            hipLaunchKernelGGL(split_reduce_kernel<true>, dim3((unsigned)((n + 255) / 256)),
                               dim3(256), 0, st, gu, s.El);
            e = hipGetLastError();
          }
        } else {
          e = launch_gemm<1, 1, 2, 4, true, 16, 64, 4, 1>(gu, mt * gu.n_tiles_n, env, st);
        }
        if (e == hipSuccess && ev) e = hipEventRecord(ev[1], st);
        if (e == hipSuccess) e = launch_gemm<1, 1, 2, 4, false, 16, 64, 4, 1>(dn, mt * dn.n_tiles_n, env, st);
      }
      break;
    case Plan::kDecode64:
      gu.n_tiles_n = ntn(s.F, 128);
      dn.n_tiles_n = ntn(s.d, 256);
      e = launch_gemm<2, 1, 2, 4, true, 16, 64, 4, 1>(gu, mt * gu.n_tiles_n, env, st);
      if (e == hipSuccess && ev) e = hipEventRecord(ev[1], st);
      if (e == hipSuccess) e = launch_gemm<2, 1, 2, 4, false, 16, 64, 4, 1>(dn, mt * dn.n_tiles_n, env, st);
      break;
    case Plan::kFp8:
      gu.n_tiles_n = ntn(s.F, 256);
      dn.n_tiles_n = ntn(s.d, 512);
      e = launch_prefill<4, 1, 2, 8, true, 8, 64, 2, 1>(gu, mt * gu.n_tiles_n, env, st);
      if (e == hipSuccess && ev) e = hipEventRecord(ev[1], st);
      if (e == hipSuccess) e = launch_prefill<4, 1, 2, 8, false, 8, 64, 2, 1>(dn, mt * dn.n_tiles_n, env, st);
      break;
    case Plan::kWide:
      gu.n_tiles_n = ntn(s.F, 256);
      dn.n_tiles_n = ntn(s.d, 512);
      e = launch_prefill<2, 2, 4, 4, true, 16, 64, 2, 1>(gu, mt * gu.n_tiles_n, env, st);
      if (e == hipSuccess && ev) e = hipEventRecord(ev[1], st);
      if (e == hipSuccess) e = launch_prefill<2, 2, 4, 4, false, 16, 64, 2, 1>(dn, mt * dn.n_tiles_n, env, st);
      break;
    case Plan::kBig:
      gu.n_tiles_n = ntn(s.F, 128);
      dn.n_tiles_n = ntn(s.d, 256);
      e = launch_prefill<2, 4, 4, 2, true, 16, 64, 2, 1>(gu, mt * gu.n_tiles_n, env, st);
      if (e == hipSuccess && ev) e = hipEventRecord(ev[1], st);
      if (e == hipSuccess) e = launch_prefill<2, 4, 4, 2, false, 16, 64, 2, 1>(dn, mt * dn.n_tiles_n, env, st);
      break;
    case Plan::kDecodeFp4:
      if (s.blocked) {
        // each wave streams 4 blocks (gate/up: 64 features), 2 slices of 64 K
        // ahead, two workgroups of 4 waves per CU
        gu.n_tiles_n = s.F / 64;
        dn.n_tiles_n = s.d / 128;
        e = launch_stream<true, 4, 4, 2, 2>(gu, mt * gu.n_tiles_n, env, st);
        if (e == hipSuccess && ev) e = hipEventRecord(ev[1], st);
        if (e == hipSuccess) e = launch_stream<false, 4, 4, 2, 2>(dn, mt * dn.n_tiles_n, env, st);
      } else {
        // row-major weights: staged 32 x 256 tiles, 128-deep K steps, two
        // stages, three workgroups per CU (streamed, a lane's 16-byte load
        // covers 32 B of each of 32 rows: 64.3 against 59 us for the Qwen3
        // gate/up)
        gu.n_tiles_n = ntn(s.F, 128);
        dn.n_tiles_n = ntn(s.d, 256);
        e = launch_gemm<1, 1, 2, 4, true, 4, 128, 2, 3>(gu, mt * gu.n_tiles_n, env, st);
        if (e == hipSuccess && ev) e = hipEventRecord(ev[1], st);
        if (e == hipSuccess) e = launch_gemm<1, 1, 2, 4, false, 4, 128, 2, 3>(dn, mt * dn.n_tiles_n, env, st);
      }
      break;
    case Plan::kFp4:
      gu.n_tiles_n = ntn(s.F, 256);
      dn.n_tiles_n = ntn(s.d, 512);
      e = launch_prefill<4, 1, 2, 8, true, 4, 64, 4, 1>(gu, mt * gu.n_tiles_n, env, st);
      if (e == hipSuccess && ev) e = hipEventRecord(ev[1], st);
      if (e == hipSuccess) e = launch_prefill<4, 1, 2, 8, false, 4, 64, 4, 1>(dn, mt * dn.n_tiles_n, env, st);
      break;
    case Plan::kF32:
      break;
  }
  if (e == hipSuccess && ev) e = hipEventRecord(ev[2], st);
  return e;
}

namespace {

// Blocked weight layout: thread per 16-byte chunk of the destination.  Unit
// (e, rb, ks) covers rows rb*32 .. +32 and K values ks*64 .. +64; it is
// C/2 operand loads of 1 KB (C = 16-byte chunks per unit row), load q, lane
// l holding chunk 2q + l/32 of row rb*32 + feat(l % 32), the row the MFMA
// operand of lane l reads (feat: the GEMMs' permuted feature order inside a
// 32-row block).
__global__ __launch_bounds__(256) void pack_weights_kernel(const uint4* __restrict__ src,
                                                           uint4* __restrict__ dst, int Nout,
                                                           int K, int row_bytes,
                                                           long long n_chunks) {
  const long long q = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (q >= n_chunks) return;
  const int C = row_bytes / 16;               // chunks per unit row
  const long long unit_chunks = 32LL * C;
  const int nk = K / 64;
  const long long u = q / unit_chunks;        // unit index (e, rb, ks)
  const int in = (int)(q % unit_chunks);
  const int ld = in / 64, l = in % 64;        // operand load, lane
  const int r = l & 31;
  const int c = 2 * ld + (l >> 5);            // chunk of the unit row
  const int ks = (int)(u % nk);
  const long long erb = u / nk;               // e * (Nout / 32) + rb
  const int row = (int)(erb % (Nout / 32)) * 32 +
                  ((r & ~31) | (((r >> 2) & 1) << 4) | (((r >> 3) & 3) << 2) | (r & 3));
  const long long e = erb / (Nout / 32);
  const long long src_chunk =
      ((e * Nout + row) * (long long)(K / 64) + ks) * C + c;  // K/64 units of C chunks per row
  dst[q] = src[src_chunk];
}

}  // namespace

hipError_t pack_weights(const Shape& s, int which, const void* src, void* dst, hipStream_t st) {
  const int Nout = which == 0 ? s.F : s.d;   // gate/up: [F][d]; down: [d][F]
  const int K = which == 0 ? s.d : s.F;
  const int wbits = s.weight == kBF16 ? 16 : s.weight == kFP8 ? 8 : 4;
  const int row_bytes = 64 * wbits / 8;
  const long long n_chunks = (long long)s.El * Nout * (K / 64) * (row_bytes / 16);
  if (n_chunks == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((n_chunks + 255) / 256);
  hipLaunchKernelGGL(pack_weights_kernel, dim3(blocks), dim3(256), 0, st,
                     static_cast<const uint4*>(src), static_cast<uint4*>(dst), Nout, K, row_bytes,
                     n_chunks);
  return hipGetLastError();
}

}  // namespace moe
