// moe_forward_noalloc: the whole-layer call with its scratch memory in a
// device array that the library itself holds, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).  It runs exactly moe_forward's kernels;
// only the scratch comes from here.
//
// `scratch` is a file-scope __device__ array: every GPU the library runs on
// holds its own copy, at its own address, until the process ends.  In host
// code the array's name is only a host-side stand-in, never a device address,
// so the device address is looked up once per device (hipGetSymbolAddress,
// with that device current) and only that address is ever handed to kernels.
#include <mutex>

#include "moe.h"
#include "moe_internal.h"

namespace {

constexpr size_t kScratchBytes = (size_t)MOE_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "whole 256-byte lines");

__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;

// Per device: the looked-up address of `scratch` (and the lookup's status),
// set once under call_once with that device current.
struct DeviceScratch {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
DeviceScratch g_dev[kMaxDevices];

hipError_t scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  DeviceScratch& d = g_dev[dev];
  std::call_once(d.once, [&d]() {
    void* p = nullptr;
    d.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (d.err == hipSuccess && p == nullptr) d.err = hipErrorInvalidSymbol;
    if (d.err == hipSuccess) d.ptr = p;
  });
  if (d.err != hipSuccess) return d.err;
  *out = d.ptr;
  return hipSuccess;
}

}  // namespace

extern "C" {

moe_status_t moe_forward_noalloc(const moe_problem_t* p, const moe_forward_args_t* a,
                                 void* stream) {
  const size_t need = moe_workspace_size(p, MOE_CALL_FORWARD);
  if (need == 0) {
    // an invalid problem: let moe_forward report which check failed (it
    // returns before touching any memory)
    return moe_forward(p, a, nullptr, 0, stream);
  }
  if (need > kScratchBytes) return MOE_ERR_UNSUPPORTED;
  void* ws = nullptr;
  if (scratch_ptr(&ws) != hipSuccess) return MOE_ERR_HIP;
  return moe_forward(p, a, ws, kScratchBytes, stream);
}

}  // extern "C"
