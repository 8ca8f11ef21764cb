// Read-only streaming kernel: the achievable HBM read rate for a buffer of a
// given size, measured beside the matmul kernels with the same timing method.
// Every byte of the buffer is read once with 16-byte non-temporal buffer
// loads, four independent loads in flight per thread (each wave load covers
// 1 KiB, a workgroup's four loads 16 KiB contiguous), in a grid-stride loop;
// each workgroup folds what it read into one word (XOR) and stores it, so
// nothing is optimised away and the result is checkable: the XOR of all
// stored words equals the XOR of the buffer.  Measured over 39.8 MB against
// 1, 2, 4 and 8 loads in flight and 256 to 8192 workgroups: every shape from
// 1024 workgroups up within 1% of the best (7.44 µs).
#include <hip/hip_runtime.h>

#include "qmm_device.h"
#include "qmm_internal.h"
#include "qmm_launch.h"

namespace qmm {
namespace {

__global__ __launch_bounds__(256) void stream_read_kernel(const uint8_t* __restrict__ src,
                                                          uint32_t n16, uint32_t* __restrict__ sink) {
  __shared__ uint32_t red[4];
  const __amdgpu_buffer_rsrc_t r = make_rsrc(src, n16 * 16u);
  constexpr int U = 4;   // loads in flight per thread
  uint32_t h = 0;
  for (uint32_t base = blockIdx.x * 256u * U + threadIdx.x; base < n16; base += gridDim.x * 256u * U) {
    u32x4_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // past the end: an offset beyond the buffer's range, which reads zeros
      const uint32_t i = base + 256u * u;
      v[u] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, int(i < n16 ? 16u * i : 0x80000000u), 0, 2));
    }
#pragma unroll
    for (int u = 0; u < U; ++u) h ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  // XOR over the workgroup: within the wave by shuffles, across waves in LDS
  for (int o = 32; o >= 1; o >>= 1) h ^= uint32_t(__shfl_xor(int(h), o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = h;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

}  // namespace

int launch_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  launch_kernel(stream_read_kernel, dim3(kStreamBlocks), dim3(256), s,
                static_cast<const uint8_t*>(src), uint32_t(bytes / 16), sink);
  return int(hipGetLastError());
}

}  // namespace qmm
