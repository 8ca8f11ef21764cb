// qmm_pack / qmm_unpack kernels: canonical weights <-> MI355X device layout.
// A bit/byte permutation plus a header; no arithmetic on weight values
// (format and layout in qmm_internal.h).
#include <hip/hip_runtime.h>

#include <atomic>

#include "qmm_device.h"
#include "qmm_internal.h"

namespace qmm {
namespace {

// Canonical word: nibble j holds q[8w + j].  Device word: even codes in the
// low half-word, odd codes in the high half-word (see qmm_internal.h).
__device__ __forceinline__ uint32_t to_device_word(uint32_t c) {
  uint32_t r = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r |= ((c >> (8 * i)) & 0xFu) << (4 * i);
    r |= ((c >> (8 * i + 4)) & 0xFu) << (16 + 4 * i);
  }
  return r;
}

__device__ __forceinline__ uint32_t from_device_word(uint32_t v) {
  uint32_t r = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r |= ((v >> (4 * i)) & 0xFu) << (8 * i);
    r |= ((v >> (16 + 4 * i)) & 0xFu) << (8 * i + 4);
  }
  return r;
}

// Zeroes the header block and the alignment gaps after the codes and after
// the metadata, then writes the header fields.  One block of 64 threads.
__global__ void write_header_kernel(uint8_t* packed, PackedHeader h, int64_t gap0, int64_t gap0_end,
                                    int64_t gap1, int64_t gap1_end) {
  for (int64_t i = threadIdx.x; i < kHeaderBytes; i += blockDim.x) packed[i] = 0;
  for (int64_t i = gap0 + threadIdx.x; i < gap0_end; i += blockDim.x) packed[i] = 0;
  for (int64_t i = gap1 + threadIdx.x; i < gap1_end; i += blockDim.x) packed[i] = 0;
  __syncthreads();
  if (threadIdx.x == 0) *reinterpret_cast<PackedHeader*>(packed) = h;
}

// Zero the metadata of the rows that pad n to a multiple of 4 (the last quad).
__device__ void zero_pad_rows(uint8_t* __restrict__ out_meta, const Slabs& L) {
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  const int64_t n4 = (L.n + 3) & ~int64_t(3);
  const int rmb = int(L.meta_quad() / 4), full = L.meta_full(), last = L.count() - 1;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < (n4 - L.n) * rmb; i += stride) {
    const int64_t r = L.n + i / rmb;
    const int b = int(i % rmb);
    const int s = b / full < last ? b / full : last;
    out_meta[L.meta(s, r) + (b - s * full)] = 0;
  }
}

// One thread per canonical code word (8 codes) and per metadata group; the
// word of row r holding codes [8j, 8j + 8) goes to its slab position.  A scale
// that is not finite or has magnitude 2^100 or more, or a bias that is not
// finite, flags the blob invalid (the MFMA dequantisation multiplies the scale
// by 2^24, which must stay finite).
__global__ void pack_affine_kernel(const uint32_t* __restrict__ codes,
                                   const uint16_t* __restrict__ scales,
                                   const uint16_t* __restrict__ biases,
                                   uint8_t* __restrict__ out_codes, uint8_t* __restrict__ out_meta,
                                   Slabs L, uint32_t* __restrict__ flags) {
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  const int64_t wpr = L.d / 8, gpr = L.d / 64;
  bool bad = false;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < L.n * wpr; i += stride) {
    const int64_t r = i / wpr;
    const int k = int(i % wpr) * 8;
    *reinterpret_cast<uint32_t*>(out_codes + L.code_byte(r, k)) = to_device_word(codes[i]);
  }
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < L.n * gpr; i += stride) {
    const int64_t r = i / gpr;
    const int k = int(i % gpr) * 64;
    const uint32_t sc = scales[i], bi = biases[i];
    bad |= ((sc >> 7) & 0xFFu) >= 127u + 100u || ((bi >> 7) & 0xFFu) == 0xFFu;
    *reinterpret_cast<uint32_t*>(out_meta + L.meta_byte(r, k)) = sc | (bi << 16);
  }
  zero_pad_rows(out_meta, L);
  if (bad) atomicOr(flags, kFlagInvalid);
}

__global__ void unpack_affine_kernel(const uint8_t* __restrict__ in_codes,
                                     const uint8_t* __restrict__ in_meta, uint32_t* __restrict__ codes,
                                     uint16_t* __restrict__ scales, uint16_t* __restrict__ biases,
                                     Slabs L) {
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  const int64_t wpr = L.d / 8, gpr = L.d / 64;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < L.n * wpr; i += stride) {
    const int64_t r = i / wpr;
    const int k = int(i % wpr) * 8;
    codes[i] = from_device_word(*reinterpret_cast<const uint32_t*>(in_codes + L.code_byte(r, k)));
  }
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < L.n * gpr; i += stride) {
    const int64_t r = i / gpr;
    const int k = int(i % gpr) * 64;
    const uint32_t m = *reinterpret_cast<const uint32_t*>(in_meta + L.meta_byte(r, k));
    scales[i] = uint16_t(m & 0xFFFFu);
    biases[i] = uint16_t(m >> 16);
  }
}

// MXFP4 codes keep their canonical byte order and only move to their slab
// position (16-byte pieces: 32 codes, one group); the E8M0 bytes move the same
// way, and any 255 (NaN scale) flags the blob invalid.
__global__ void pack_mxfp4_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ e8m0,
                                  uint8_t* __restrict__ out_codes, uint8_t* __restrict__ out_meta,
                                  Slabs L, uint32_t* __restrict__ flags) {
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  const int64_t gpr = L.d / 32;
  bool bad = false;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < L.n * gpr; i += stride) {
    const int64_t r = i / gpr;
    const int k = int(i % gpr) * 32;
    // the canonical array is only guaranteed 4-byte aligned
    const uint32_t* src = reinterpret_cast<const uint32_t*>(codes) + 4 * i;
    *reinterpret_cast<u32x4_t*>(out_codes + L.code_byte(r, k)) = u32x4_t{src[0], src[1], src[2], src[3]};
    const uint8_t e = e8m0[i];
    bad |= (e == 255);
    out_meta[L.meta_byte(r, k)] = e;
  }
  // zero the padding that ends each row's metadata in a narrow last slab
  const int sl = L.count() - 1;
  const int used = L.width(sl) / 32, pad = L.meta_row(sl) - used;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < L.n * pad; i += stride)
    out_meta[L.meta(sl, i / pad) + used + i % pad] = 0;
  zero_pad_rows(out_meta, L);
  if (bad) atomicOr(flags, kFlagInvalid);
}

__global__ void unpack_mxfp4_kernel(const uint8_t* __restrict__ in_codes,
                                    const uint8_t* __restrict__ in_meta, uint8_t* __restrict__ codes,
                                    uint8_t* __restrict__ e8m0, Slabs L) {
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  const int64_t gpr = L.d / 32;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < L.n * gpr; i += stride) {
    const int64_t r = i / gpr;
    const int k = int(i % gpr) * 32;
    const u32x4_t v = load16(in_codes + L.code_byte(r, k));
    uint32_t* dst = reinterpret_cast<uint32_t*>(codes) + 4 * i;
    dst[0] = v[0];
    dst[1] = v[1];
    dst[2] = v[2];
    dst[3] = v[3];
    e8m0[i] = in_meta[L.meta_byte(r, k)];
  }
}

int grid_for(int64_t items) {
  int64_t g = (items + 255) / 256;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return int(g);
}

}  // namespace

int device_info(DevInfo* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return int(e);
  // per-device cache, safe under concurrent callers (a racing first query
  // stores the same value twice)
  static std::atomic<int> cached_cus[64];
  int cus = dev >= 0 && dev < 64 ? cached_cus[dev].load(std::memory_order_relaxed) : 0;
  if (cus <= 0) {
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return int(e);
    if (dev >= 0 && dev < 64) cached_cus[dev].store(cus, std::memory_order_relaxed);
  }
  out->cus = cus;
  return 0;
}

int launch_pack(int f, int64_t n, int64_t d, const void* codes, const void* scales,
                const void* biases, void* packed, void* stream) {
  Layout l;
  if (!layout_of(f, n, d, &l)) return int(hipErrorInvalidValue);
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* p = static_cast<uint8_t*>(packed);
  PackedHeader h{kMagic, kLayoutVersion, uint32_t(f), 0u, n, d, l.codes_offset, l.meta_offset,
                 l.total_bytes};
  hipLaunchKernelGGL(write_header_kernel, dim3(1), dim3(64), 0, s, p, h,
                     l.codes_offset + n * (d / 2), l.meta_offset, l.meta_offset + l.meta_bytes,
                     l.total_bytes);
  const Slabs L{n, int(d), f};
  if (f == QMM_AFFINE4_G64) {
    hipLaunchKernelGGL(pack_affine_kernel, dim3(grid_for(n * (d / 8))), dim3(256), 0, s,
                       static_cast<const uint32_t*>(codes), static_cast<const uint16_t*>(scales),
                       static_cast<const uint16_t*>(biases), p + l.codes_offset, p + l.meta_offset, L,
                       reinterpret_cast<uint32_t*>(p + offsetof(PackedHeader, flags)));
  } else {
    hipLaunchKernelGGL(pack_mxfp4_kernel, dim3(grid_for(n * (d / 32))), dim3(256), 0, s,
                       static_cast<const uint8_t*>(codes), static_cast<const uint8_t*>(scales),
                       p + l.codes_offset, p + l.meta_offset, L,
                       reinterpret_cast<uint32_t*>(p + offsetof(PackedHeader, flags)));
  }
  return int(hipGetLastError());
}

int read_header(const void* packed, PackedHeader* out, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(out, packed, sizeof(PackedHeader), hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return int(e);
  return int(hipStreamSynchronize(s));
}

int launch_unpack(int f, int64_t n, int64_t d, const void* packed, void* codes, void* scales,
                  void* biases, void* stream) {
  Layout l;
  if (!layout_of(f, n, d, &l)) return int(hipErrorInvalidValue);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint8_t* p = static_cast<const uint8_t*>(packed);
  const Slabs L{n, int(d), f};
  if (f == QMM_AFFINE4_G64) {
    hipLaunchKernelGGL(unpack_affine_kernel, dim3(grid_for(n * (d / 8))), dim3(256), 0, s,
                       p + l.codes_offset, p + l.meta_offset, static_cast<uint32_t*>(codes),
                       static_cast<uint16_t*>(scales), static_cast<uint16_t*>(biases), L);
  } else {
    hipLaunchKernelGGL(unpack_mxfp4_kernel, dim3(grid_for(n * (d / 32))), dim3(256), 0, s,
                       p + l.codes_offset, p + l.meta_offset, static_cast<uint8_t*>(codes),
                       static_cast<uint8_t*>(scales), L);
  }
  return int(hipGetLastError());
}

}  // namespace qmm
