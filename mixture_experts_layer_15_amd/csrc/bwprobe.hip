// Measurement helper (not part of the layer): an HBM read stream and a plain
// copy with 16-byte accesses over 2 GiB buffers.  It gives the achievable
// bandwidth on the box, and the copy kernel of known size that calibrates the
// FETCH_SIZE / WRITE_SIZE counters (bytes moved per dispatch are known
// exactly: 2 GiB read, 2 GiB written).  Mode "lds": how fast LDS-DMA
// (buffer_load_dwordx4 ... lds) fills the expert GEMMs' 64 KB stages, one
// 8-wave workgroup per CU with a 2-stage ring and no compute, from data read
// once (HBM) and from a 1 MB region per XCD that all its workgroups read (L2).
#include <hip/hip_runtime.h>
#include <cstdio>
#include <cstdlib>
#include <cstring>
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
#define CK(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { printf("HIP error %s at %d\n", hipGetErrorString(e_), __LINE__); exit(1);} } while (0)

__global__ void read_kernel(const u32x4* __restrict__ a, size_t n, unsigned* out) {
  size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  size_t stride = (size_t)gridDim.x * blockDim.x;
  u32x4 acc = {0, 0, 0, 0};
  for (; i < n; i += stride) acc ^= __builtin_nontemporal_load(a + i);
  unsigned v = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (v == 0x12345678u) out[0] = v;  // keeps the loads live; practically never stores
}
__global__ void copy_kernel(const u32x4* __restrict__ a, u32x4* __restrict__ b, size_t n) {
  size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  size_t stride = (size_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) b[i] = a[i];
}
constexpr int kFillThreads = 512;
constexpr int kFillStage = 65536;
constexpr int kFillLoads = kFillStage / (1024 * (kFillThreads / 64));  // 1 KB loads per wave

template <int N>
__device__ __forceinline__ void fill_wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup b streams nst stages from its region (l2: region b % 8 of 1 MB,
// wrapped; else its own nst * 64 KB) into LDS; a buffer resource bounds
// every load to the region.
template <bool kL2>
__global__ __launch_bounds__(kFillThreads, 1) void fill_kernel(const unsigned char* src,
                                                               size_t bytes, int nst,
                                                               unsigned* out) {
  extern __shared__ __align__(16) unsigned char lds[];
  const int wave = threadIdx.x / 64, l = threadIdx.x % 64;
  const size_t region = kL2 ? ((size_t)1 << 20) : (size_t)nst * kFillStage;
  const size_t base = kL2 ? (size_t)(blockIdx.x % 8) * region : (size_t)blockIdx.x * region;
  if (base + region > bytes) return;
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<unsigned char*>(src + base), (short)0, (int)region, 0x00020000);
  auto issue = [&](int st) {
    unsigned char* buf = lds + (st & 1) * kFillStage;
    const unsigned so = (unsigned)(((size_t)st * kFillStage) % region);
#pragma unroll
    for (int i = 0; i < kFillLoads; ++i) {
      const unsigned o = (wave * kFillLoads + i) * 1024;
#if defined(__HIP_DEVICE_COMPILE__)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(buf + o),
                                               16, o + 16 * l, so, 0, 0);
#else
      (void)buf; (void)o; (void)so;
#endif
    }
  };
  unsigned acc = 0;
  issue(0);
  for (int st = 0; st < nst; ++st) {
    if (st + 1 < nst) {
      issue(st + 1);
      fill_wait_vm<kFillLoads>();  // stage st landed
    } else {
      fill_wait_vm<0>();
    }
    __builtin_amdgcn_s_barrier();
    acc += lds[(st & 1) * kFillStage + threadIdx.x * 16];
    __builtin_amdgcn_s_barrier();  // nobody reads stage st's buffer any more
  }
  if (acc == 0x12345678u) out[0] = acc;
}

template <bool kL2>
double fill_rate(const unsigned char* src, size_t bytes, int nst, unsigned* out, int cu) {
  CK(hipFuncSetAttribute(reinterpret_cast<const void*>(fill_kernel<kL2>),
                         hipFuncAttributeMaxDynamicSharedMemorySize, 2 * kFillStage));
  hipEvent_t e0, e1;
  CK(hipEventCreate(&e0)); CK(hipEventCreate(&e1));
  hipLaunchKernelGGL(fill_kernel<kL2>, dim3(cu), dim3(kFillThreads), 2 * kFillStage, 0, src, bytes,
                     nst, out);
  CK(hipEventRecord(e0));
  const int iters = 5;
  for (int i = 0; i < iters; ++i)
    hipLaunchKernelGGL(fill_kernel<kL2>, dim3(cu), dim3(kFillThreads), 2 * kFillStage, 0, src,
                       bytes, nst, out);
  CK(hipEventRecord(e1)); CK(hipEventSynchronize(e1));
  float ms; CK(hipEventElapsedTime(&ms, e0, e1));
  return (double)cu * nst * kFillStage * iters / (ms * 1e-3) / 1e9;
}

int main(int argc, char** argv) {
  const char* mode = argc > 1 ? argv[1] : "both";
  const size_t bytes = (size_t)2 << 30;  // 2 GiB per buffer
  const size_t n = bytes / 16;
  u32x4 *a, *b; unsigned* out;
  CK(hipMalloc(&a, bytes)); CK(hipMalloc(&b, bytes)); CK(hipMalloc(&out, 64));
  CK(hipMemset(a, 1, bytes)); CK(hipMemset(b, 0, bytes));
  int cu = 0; CK(hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, 0));
  hipEvent_t e0, e1; CK(hipEventCreate(&e0)); CK(hipEventCreate(&e1));
  const int iters = 10;
  for (int blocks_per_cu : {4, 8, 16}) {
    dim3 grid(cu * blocks_per_cu), blk(256);
    if (!strcmp(mode, "both") || !strcmp(mode, "read")) {
      hipLaunchKernelGGL(read_kernel, grid, blk, 0, 0, a, n, out);
      CK(hipEventRecord(e0));
      for (int i = 0; i < iters; ++i) hipLaunchKernelGGL(read_kernel, grid, blk, 0, 0, a, n, out);
      CK(hipEventRecord(e1)); CK(hipEventSynchronize(e1));
      float ms; CK(hipEventElapsedTime(&ms, e0, e1));
      printf("read  blocks/CU=%2d: %.1f GB/s\n", blocks_per_cu, bytes * iters / (ms * 1e-3) / 1e9);
    }
    if (!strcmp(mode, "both") || !strcmp(mode, "copy")) {
      hipLaunchKernelGGL(copy_kernel, grid, blk, 0, 0, a, b, n);
      CK(hipEventRecord(e0));
      for (int i = 0; i < iters; ++i) hipLaunchKernelGGL(copy_kernel, grid, blk, 0, 0, a, b, n);
      CK(hipEventRecord(e1)); CK(hipEventSynchronize(e1));
      float ms; CK(hipEventElapsedTime(&ms, e0, e1));
      printf("copy  blocks/CU=%2d: %.1f GB/s (read+write)\n", blocks_per_cu, 2.0 * bytes * iters / (ms * 1e-3) / 1e9);
    }
  }
  if (!strcmp(mode, "both") || !strcmp(mode, "lds")) {
    const int nst = (int)(bytes / ((size_t)cu * kFillStage));  // each workgroup's share, read once
    const double hbm = fill_rate<false>(reinterpret_cast<const unsigned char*>(a), bytes, nst, out, cu);
    const double l2 = fill_rate<true>(reinterpret_cast<const unsigned char*>(a), bytes, nst, out, cu);
    printf("lds-dma stage fill, one 8-wave workgroup per CU: from HBM %.1f GB/s, from L2 %.1f GB/s "
           "(%.1f GB/s per CU)\n", hbm, l2, l2 / cu);
  }
  CK(hipDeviceSynchronize());
  printf("probe done, CUs=%d, bytes per buffer=%zu\n", cu, bytes);
  return 0;
}
