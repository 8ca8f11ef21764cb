// A fixed scratch area for qmm_gemm_noalloc: what qmm_gemm keeps in its
// workspace (the fp32 partial sums of the GEMM split along K; for affine
// weights through the tile kernel the fp16 activations and the operand
// exponents) lives in a file-scope device array instead, for callers that
// cannot allocate device memory.
//
// The array is part of this library's code object, so every GPU the library
// runs on holds its own copy, at its own address, until the process ends.  In
// host code `scratch` names a host-side stand-in, not that address: the device
// address is asked for once per device (hipGetSymbolAddress, with the device
// current) and only that address is ever handed to kernels.
//
// Every call on a GPU shares that GPU's array and finds the previous call's
// contents in it.  Every kernel writes what it later reads (each split-K
// workgroup stores its whole [t][256-column] block of its plane, the
// activation pre-pass every converted row and exponent), so nothing has to
// start at zero.  Calls that overlap on one GPU (different
// streams, or threads that do not order their calls) race on the array.
#include <hip/hip_runtime.h>

#include <mutex>

#include "qmm_internal.h"
#include "qmm_skinny.h"

namespace qmm {
namespace {

constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

int noalloc_scratch(void* stream, void** out) {
  int dev = 0;
  hipError_t e = stream ? hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return int(e);
  if (dev < 0 || dev >= kMaxDevices) return int(hipErrorInvalidDevice);
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    int cur = 0;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return int(e);
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return int(e);
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    const hipError_t back = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) return int(e);
    if (back != hipSuccess) return int(back);
    if (!p || reinterpret_cast<uintptr_t>(p) % 256) return int(hipErrorInvalidSymbol);
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return 0;
}

}  // namespace qmm
