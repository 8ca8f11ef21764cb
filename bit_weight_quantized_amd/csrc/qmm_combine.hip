// MoE combine: each token's expert outputs, weighted and summed back into
// token space -- the weighted scatter-add of "Colibri Kimi K3 Metal 后端实现全解析"
// (Phase 6), with the chosen experts' sigmoid weights renormalised to sum to
// one ("Kimi K3 迁移到 Google TPU 的可行性评估（v2）", §2 模型解剖: sigmoid +
// renormalize).
//
// Written as a gather, one workgroup per token, so no two threads add into the
// same output and the order of the additions is fixed (slot order): for slot j
// of token t (expert e = topk[t, j]) the row of t in e's segment is found by
// binary search (a segment lists its tokens ascending), the weight is
// weights[t, e] / Σ_j' weights[t, topk[t, j']] (summed in slot order by one
// thread), and out[t, c] = Σ_j w_j·o[row_j, c] in fp32, rounded once to bf16.
// Each thread owns 8 consecutive columns (one 16-byte load per slot).
#include <hip/hip_runtime.h>

#include <math.h>

#include "qmm_device.h"
#include "qmm_internal.h"
#include "qmm_launch.h"

namespace qmm {
namespace {

__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ o, int m_total,
                                                      int d, int k, const int32_t* __restrict__ topk,
                                                      const float* __restrict__ weights, int ne,
                                                      const int32_t* __restrict__ seg_offsets,
                                                      const int32_t* __restrict__ row_index,
                                                      uint16_t* __restrict__ out) {
  __shared__ float wj[kCombineMaxK];
  __shared__ int32_t row[kCombineMaxK];
  __shared__ float total;
  __shared__ int bad;
  const int tok = blockIdx.x;
  const int tid = threadIdx.x;
  if (tid == 0) bad = 0;
  __syncthreads();
  if (tid < k) {
    const int e = topk[int64_t(tok) * k + tid];
    float w = __builtin_nanf("");
    int r = -1;
    if (e >= 0 && e < ne) {
      w = weights[int64_t(tok) * ne + e];
      int lo = min(max(seg_offsets[e], 0), m_total);
      const int hi = min(max(seg_offsets[e + 1], lo), m_total);
      int len = hi - lo;
      while (len > 0) {   // first row in [lo, hi) whose token is >= tok
        const int half = len >> 1;
        if (row_index[lo + half] < tok) {
          lo += half + 1;
          len -= half + 1;
        } else {
          len = half;
        }
      }
      if (lo < hi && row_index[lo] == tok) r = lo;
    }
    if (r < 0) atomicOr(&bad, 1);
    wj[tid] = w;
    row[tid] = r;
  }
  __syncthreads();
  if (tid == 0) {
    float sum = 0.f;
    for (int j = 0; j < k; ++j) sum += wj[j];
    total = sum;
  }
  __syncthreads();
  if (tid < k) wj[tid] = wj[tid] / total;
  __syncthreads();
  const bool broken = bad != 0;   // a slot with no row: the token's outputs are NaN
  uint16_t* dst = out + int64_t(tok) * d;
  for (int c8 = tid; c8 < d / 8; c8 += 256) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (!broken) {
      for (int j = 0; j < k; ++j) {
        const float w = wj[j];
        const u32x4_t v = load16(o + int64_t(row[j]) * d + 8 * c8);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[2 * q] = fmaf(w, bf16_lo(v[q]), acc[2 * q]);
          acc[2 * q + 1] = fmaf(w, bf16_hi(v[q]), acc[2 * q + 1]);
        }
      }
    }
    u32x4_t pk;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float a = broken ? __builtin_nanf("") : acc[2 * q];
      const float b = broken ? __builtin_nanf("") : acc[2 * q + 1];
      pk[q] = uint32_t(f32_to_bf16(a)) | (uint32_t(f32_to_bf16(b)) << 16);
    }
    *reinterpret_cast<u32x4_t*>(dst + 8 * c8) = pk;
  }
}

}  // namespace

int launch_combine(const CombineArgs& a, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  launch_kernel(combine_kernel, dim3(unsigned(a.t)), dim3(256), s, a.o, a.m_total, a.d, a.k, a.topk,
                a.weights, a.ne, a.seg_offsets, a.row_index, a.out);
  return int(hipGetLastError());
}

}  // namespace qmm
