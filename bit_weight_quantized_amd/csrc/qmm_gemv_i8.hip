// Deferred-dequantisation decode GEMV (affine weights, int8 activations):
// "LLM Decode / Prefill 优化案例（Metal）", Step 2.  The activation row is
// quantised per row by its absolute maximum (s = absmax/127, x_q =
// round-half-even(x/s), both in fp32), the 4-bit codes meet it in exact
// integer sums (v_dot4_i32_i8, four int8 products per instruction), and scale
// and bias are applied once per 32-code chunk: scale·isum + bias·Σx_q, times
// s at the end.  An approximation of Y = X·Ŵᵀ (the activations lose bits);
// the oracle follows the same steps.
//
// Each workgroup first issues its first slabs of code loads, then quantises
// the whole row into LDS itself (the absmax, then the codes; x is held in
// registers between the two up to d = 8192), storing each 8-code piece in
// the byte order the regrouped code words unpack to -- (x0, x4, x1, x5) for
// w & 0x0F0F0F0F and (x2, x6, x3, x7) for (w >> 4) & 0x0F0F0F0F -- plus one
// int32 sum per 32-code chunk.  Then, as in the bf16 GEMV, a wave owns 4 rows,
// lane (row, chunk) handles 32 codes of one row per slab, and a ring of three
// slabs of code loads (issued unconditionally, in the order they are used) is
// in flight per lane; the chunk's group metadata comes with its slab.
#include <hip/hip_runtime.h>

#include <math.h>

#include "qmm_deferred.h"
#include "qmm_device.h"
#include "qmm_internal.h"
#include "qmm_launch.h"

namespace qmm {
namespace {

constexpr int kI8Waves = 4;
constexpr int kI8Ring = 3;
constexpr int kI8XC = 4;    // activation pieces per thread kept in registers (d <= 8192)
constexpr uint32_t kOOB = 0x80000000u;   // OR-ed into a buffer offset: past every range

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__global__ __launch_bounds__(64 * kI8Waves) void gemv_i8_kernel(const uint8_t* __restrict__ codes,
                                                                 const uint8_t* __restrict__ meta,
                                                                 uint32_t codes_bytes,
                                                                 uint32_t meta_bytes, int n, int d,
                                                                 const uint16_t* __restrict__ x,
                                                                 uint16_t* __restrict__ y) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  // LDS: x_q bytes [d], then one int32 sum per 32-code chunk, then 4 floats
  int8_t* xq = reinterpret_cast<int8_t*>(smem);
  int32_t* xsum = reinterpret_cast<int32_t*>(smem + d);
  float* red = reinterpret_cast<float*>(smem + d + 4 * (d / 32));

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int npieces = d / 8;

  // 0. the first slabs of this lane's codes and metadata, issued before the
  //    activation work so their memory latency runs under it (a wave owns 4
  //    rows; lane = (row rsub, chunk c) of each slab)
  const Slabs L{n, d, QMM_AFFINE4_G64};
  const int nslabs = L.count();
  const int rsub = lane >> 4, c = lane & 15;
  const int quad = blockIdx.x * kI8Waves + wave;
  const int row = quad * 4 + rsub;
  const int lrow = min(row, n - 1);   // rows past n (last quad only) load row n - 1, store nothing
  const __amdgpu_buffer_rsrc_t cr = make_rsrc(codes, codes_bytes);
  const __amdgpu_buffer_rsrc_t mr = make_rsrc(meta, meta_bytes);
  auto code_off = [&](int s) -> uint32_t {
    if (s >= nslabs) return kOOB;
    return 32 * c < L.width(s) ? uint32_t(L.codes(s, lrow)) + 16u * c : kOOB;
  };
  auto meta_off = [&](int s) -> uint32_t {
    if (s >= nslabs) return kOOB;
    return 32 * c < L.width(s) ? uint32_t(L.meta(s, lrow)) + 4u * (c >> 1) : kOOB;
  };
  u32x4_t ring[kI8Ring];
  uint32_t mring[kI8Ring];
#pragma unroll
  for (int j = 0; j < kI8Ring; ++j) {
    ring[j] = buf_load16(cr, code_off(j));
    mring[j] = buf_load4(mr, meta_off(j));
  }

  // 1. absmax of the row; the first kI8XC pieces per thread stay in registers
  //    for the quantisation (all of them for d <= 8192), the rest are re-read
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, uint32_t(d) * 2u);
  u32x4_t xc[kI8XC];
#pragma unroll
  for (int u = 0; u < kI8XC; ++u) xc[u] = buf_load16(xr, 16u * uint32_t(tid + 64 * kI8Waves * u));   // past d: zeros
  float amax = 0.f;
#pragma unroll
  for (int u = 0; u < kI8XC; ++u)
#pragma unroll
    for (int q = 0; q < 4; ++q) amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(xc[u][q])), fabsf(bf16_hi(xc[u][q]))));
  for (int i = tid + 64 * kI8Waves * kI8XC; i < npieces; i += 64 * kI8Waves) {
    const u32x4_t v = load16(x + 8 * i);
#pragma unroll
    for (int q = 0; q < 4; ++q) amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(v[q])), fabsf(bf16_hi(v[q]))));
  }
  amax = wave_max(amax);
  if (lane == 0) red[wave] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float sx = amax / 127.0f;

  // 2. codes of the row, in the byte order the weight words unpack to
  auto qz = [&](float v) -> uint32_t {
    const int q = sx > 0.f ? int(rintf(v / sx)) : 0;
    return uint32_t(q) & 0xFFu;
  };
  auto put = [&](int i, const u32x4_t& v) {
    // v[q] holds elements 2q (low) and 2q + 1 (high)
    const uint32_t e0 = qz(bf16_lo(v[0])), e1 = qz(bf16_hi(v[0])), e2 = qz(bf16_lo(v[1])), e3 = qz(bf16_hi(v[1]));
    const uint32_t e4 = qz(bf16_lo(v[2])), e5 = qz(bf16_hi(v[2])), e6 = qz(bf16_lo(v[3])), e7 = qz(bf16_hi(v[3]));
    uint32_t* dst = reinterpret_cast<uint32_t*>(xq + 8 * i);
    dst[0] = e0 | (e4 << 8) | (e1 << 16) | (e5 << 24);
    dst[1] = e2 | (e6 << 8) | (e3 << 16) | (e7 << 24);
  };
#pragma unroll
  for (int u = 0; u < kI8XC; ++u) {
    const int i = tid + 64 * kI8Waves * u;
    if (i < npieces) put(i, xc[u]);
  }
  for (int i = tid + 64 * kI8Waves * kI8XC; i < npieces; i += 64 * kI8Waves) put(i, load16(x + 8 * i));
  __syncthreads();
  for (int cc = tid; cc < d / 32; cc += 64 * kI8Waves) {
    int sum = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      sum = __builtin_amdgcn_sdot4(reinterpret_cast<const int32_t*>(xq + 32 * cc)[j], 0x01010101, sum, false);
    xsum[cc] = sum;
  }
  __syncthreads();

  // 3. the integer GEMV over the slabs, three in flight per lane
  float acc = 0.f;
  for (int s0 = 0; s0 < nslabs; s0 += kI8Ring) {
#pragma unroll
    for (int j = 0; j < kI8Ring; ++j) {
      const int s = s0 + j;
      if (s < nslabs && 32 * c < L.width(s)) {
        const int chunk = s * 16 + c;
        const int32_t* xp = reinterpret_cast<const int32_t*>(xq + 32 * chunk);
        int isum = 0;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          isum = __builtin_amdgcn_sdot4(int(ring[j][w] & 0x0F0F0F0Fu), xp[2 * w], isum, false);
          isum = __builtin_amdgcn_sdot4(int((ring[j][w] >> 4) & 0x0F0F0F0Fu), xp[2 * w + 1], isum, false);
        }
        acc += bf16_lo(mring[j]) * float(isum) + bf16_hi(mring[j]) * float(xsum[chunk]);
      }
      ring[j] = buf_load16(cr, code_off(s + kI8Ring));
      mring[j] = buf_load4(mr, meta_off(s + kI8Ring));
    }
  }
  // 4. sum the row's 16 lanes, scale once
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
  if (c == 0 && row < n) y[row] = f32_to_bf16(acc * sx);
}

}  // namespace

int launch_gemv_i8(const GemvArgs& a, void* stream) {
  Layout l;
  if (!layout_of(QMM_AFFINE4_G64, a.n, a.d, &l)) return int(hipErrorInvalidValue);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int quads = (a.n + 3) / 4;
  const dim3 grid(unsigned((quads + kI8Waves - 1) / kI8Waves));
  const size_t lds = size_t(a.d) + 4 * size_t(a.d / 32) + 16;
  launch_kernel_lds(gemv_i8_kernel, grid, dim3(64 * kI8Waves), lds, s, a.packed + l.codes_offset,
                    a.packed + l.meta_offset, uint32_t(int64_t(a.n) * (a.d / 2)), uint32_t(l.meta_bytes),
                    a.n, a.d, a.x, a.y);
  return int(hipGetLastError());
}

}  // namespace qmm
