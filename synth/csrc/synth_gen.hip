// GPU twin of synth/__init__.py for the integer streams (codes and E8M0
// bytes): SplitMix64 in counter mode, bit-identical to the numpy version.
// Used to fill the routed-expert weight stacks (about 15.7 GB for 896
// experts) directly in device memory.  Only integer arithmetic, so host and
// device agree bit for bit.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;
constexpr uint64_t kM1 = 0xBF58476D1CE4E5B9ull;
constexpr uint64_t kM2 = 0x94D049BB133111EBull;
constexpr uint64_t kK0 = 0x243F6A8885A308D3ull;

__host__ __device__ inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * kM1;
  z = (z ^ (z >> 27)) * kM2;
  return z ^ (z >> 31);
}

// dst[j] = byte (start_byte + j) of the little-endian stream of h(i).
// Whole 8-byte hashes per thread; the byte range may start and end anywhere.
__global__ void code_bytes_kernel(uint64_t key, uint8_t* __restrict__ dst, int64_t nbytes,
                                  int64_t start_byte) {
  const int64_t h0 = start_byte / 8;
  const int64_t h1 = (start_byte + nbytes + 7) / 8;
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t h = h0 + int64_t(blockIdx.x) * blockDim.x + threadIdx.x; h < h1; h += stride) {
    const uint64_t v = mix64(key + uint64_t(h + 1) * kGamma);
    const int64_t b0 = h * 8 - start_byte;
    if (b0 >= 0 && b0 + 8 <= nbytes && ((reinterpret_cast<uintptr_t>(dst) + b0) & 7) == 0) {
      *reinterpret_cast<uint64_t*>(dst + b0) = v;
    } else {
      for (int i = 0; i < 8; ++i) {
        const int64_t b = b0 + i;
        if (b >= 0 && b < nbytes) dst[b] = uint8_t(v >> (8 * i));
      }
    }
  }
}

// dst[i] = lo + ((h(start + i) >> 32) * m >> 32), i < count
__global__ void small_int_u8_kernel(uint64_t key, uint8_t* __restrict__ dst, int64_t count,
                                    int64_t start, uint32_t lo, uint32_t m) {
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < count; i += stride) {
    const uint64_t v = mix64(key + uint64_t(start + i + 1) * kGamma);
    dst[i] = uint8_t(lo + uint32_t(((v >> 32) * m) >> 32));
  }
}

int grid_for(int64_t items) {
  int64_t g = (items + 255) / 256;
  if (g > 65536) g = 65536;
  return g < 1 ? 1 : int(g);
}

}  // namespace

extern "C" {

uint64_t synth_key(uint32_t seed, uint32_t stream, uint32_t sub) {
  return mix64((uint64_t(seed) << 32) ^ (uint64_t(stream) << 20) ^ uint64_t(sub) ^ kK0);
}

// Returns a hipError_t (0 = success).  Asynchronous on `stream`.
int synth_code_bytes(uint32_t seed, uint32_t stream_id, uint32_t sub, void* dst, int64_t nbytes,
                     int64_t start_byte, void* stream) {
  if (!dst || nbytes < 0 || start_byte < 0 || stream_id >= (1u << 12) || sub >= (1u << 20))
    return int(hipErrorInvalidValue);
  if (nbytes == 0) return 0;
  hipLaunchKernelGGL(code_bytes_kernel, dim3(grid_for((nbytes + 7) / 8 + 1)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), synth_key(seed, stream_id, sub),
                     static_cast<uint8_t*>(dst), nbytes, start_byte);
  return int(hipGetLastError());
}

int synth_small_int_u8(uint32_t seed, uint32_t stream_id, uint32_t sub, void* dst, int64_t count,
                       int64_t start, uint32_t lo, uint32_t m, void* stream) {
  if (!dst || count < 0 || start < 0 || m == 0 || lo + m > 256 || stream_id >= (1u << 12) ||
      sub >= (1u << 20))
    return int(hipErrorInvalidValue);
  if (count == 0) return 0;
  hipLaunchKernelGGL(small_int_u8_kernel, dim3(grid_for(count)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), synth_key(seed, stream_id, sub),
                     static_cast<uint8_t*>(dst), count, start, lo, m);
  return int(hipGetLastError());
}

}  // extern "C"
