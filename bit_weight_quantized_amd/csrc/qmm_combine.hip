// MoE combine: each token's expert outputs, weighted and summed back into
// token space -- the weighted scatter-add of "Colibri Kimi K3 Metal 后端实现全解析"
// (Phase 6), with the chosen experts' sigmoid weights renormalised to sum to
// one ("Kimi K3 迁移到 Google TPU 的可行性评估（v2）", §2 模型解剖: sigmoid +
// renormalize).
//
// Written as a gather, one workgroup per token and 2048-column block, so no
// two threads add into the same output and the order of the additions is
// fixed (slot order): for slot j of token t (expert e = topk[t, j]) the row of
// t in e's segment is found by search (a segment lists its tokens ascending),
// the weight is weights[t, e] / Σ_j' weights[t, topk[t, j']] (summed in slot
// order by one thread), and out[t, c] = Σ_j w_j·o[row_j, c] in fp32, rounded
// once to bf16.  Each thread owns 8 consecutive columns (one 16-byte load per
// slot).
//
// Latency, not bytes, is what this kernel has to fight: the row search is a
// chain of dependent loads before the first expert row can be read.  Each slot
// gets P lanes (P a power of two, 256/k rounded down, at most a wave), which
// probe P evenly spaced entries of the remaining range at once; a ballot counts
// the probes below the token and narrows the range to one gap, so a segment of
// up to P entries takes one round trip and one of up to P² two (a lane-serial
// binary search takes log2 of the length).  The expert rows are then read 16
// slots at a time, all 16 loads issued before the first is used.
#include <hip/hip_runtime.h>

#include <limits.h>
#include <math.h>

#include <type_traits>

#include "qmm_device.h"
#include "qmm_internal.h"
#include "qmm_launch.h"

namespace qmm {
namespace {

constexpr int kCombineCols = 256 * 8;   // output columns per workgroup
constexpr int kSlotBatch = 16;          // expert-row loads in flight per thread

// bits of `mask` belonging to the P-lane group that holds lane `lane`
__device__ __forceinline__ uint64_t group_bits(uint64_t mask, int lane, int p) {
  const uint64_t m = p == 64 ? ~0ull : ((1ull << p) - 1ull);
  return (mask >> (lane & ~(p - 1))) & m;
}

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
  const int lane = tid & 63;
  if (tid == 0) bad = 0;
  __syncthreads();

  // 1. the row of every slot: P lanes per slot
  int p = 64;
  while (p * k > 256) p >>= 1;   // k <= 64, so p >= 4
  const int j = tid / p, i = tid & (p - 1);
  if (j < k) {
    const int e = topk[int64_t(tok) * k + j];
    float w = __builtin_nanf("");
    int r = -1;
    if (e >= 0 && e < ne) {
      w = weights[int64_t(tok) * ne + e];
      int lo = min(max(seg_offsets[e], 0), m_total);
      int hi = min(max(seg_offsets[e + 1], lo), m_total);
      // invariant: entries before lo are < tok; the first entry >= tok, if
      // any, lies in [lo, hi)
      while (hi - lo > p) {   // uniform over the slot's lanes
        const int step = (hi - lo + p - 1) / p;
        const int q = lo + i * step;
        const bool below = q < hi && row_index[q] < tok;
        const int c = __popcll(group_bits(__ballot(below), lane, p));   // a prefix of the probes
        if (c == 0) {
          hi = lo + 1;
        } else {
          const int last = lo + (c - 1) * step;        // the last probe below tok
          const int next = last + step;                // the first probe not below it
          lo = last + 1;
          hi = min(hi, next + 1);
        }
      }
      const int q = lo + i;
      const uint64_t hit = group_bits(__ballot(q < hi && row_index[q] == tok), lane, p);
      if (hit) r = lo + __builtin_ctzll(hit);
    }
    if (i == 0) {
      if (r < 0) atomicOr(&bad, 1);
      wj[j] = w;
      row[j] = r;
    }
  }
  __syncthreads();
  if (tid == 0) {
    float sum = 0.f;
    for (int jj = 0; jj < k; ++jj) sum += wj[jj];
    total = sum;
  }
  __syncthreads();
  if (tid < k) wj[tid] = wj[tid] / total;
  __syncthreads();

  // 2. the weighted sum of the token's expert rows in slot order, in batches
  //    of 16, then 4, then 1 slots: every load of a batch is issued before
  //    the first is used (no guard inside a batch, which would let the
  //    compiler move each load next to its use)
  const bool broken = bad != 0;   // a slot with no row: the token's outputs are NaN
  const int c8 = blockIdx.y * (kCombineCols / 8) + tid;
  if (c8 >= d / 8) return;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (!broken) {
    const uint16_t* col = o + 8 * int64_t(c8);
    auto batch = [&](auto nb, int j0) {
      constexpr int B = decltype(nb)::value;
      u32x4_t v[B];
#pragma unroll
      for (int u = 0; u < B; ++u) v[u] = load16(col + int64_t(row[j0 + u]) * d);
#pragma unroll
      for (int u = 0; u < B; ++u) {
        const float w = wj[j0 + u];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[2 * q] = fmaf(w, bf16_lo(v[u][q]), acc[2 * q]);
          acc[2 * q + 1] = fmaf(w, bf16_hi(v[u][q]), acc[2 * q + 1]);
        }
      }
    };
    int j0 = 0;
    for (; j0 + kSlotBatch <= k; j0 += kSlotBatch) batch(std::integral_constant<int, kSlotBatch>{}, j0);
    for (; j0 + 4 <= k; j0 += 4) batch(std::integral_constant<int, 4>{}, j0);
    for (; j0 < k; ++j0) batch(std::integral_constant<int, 1>{}, j0);
  }
  u32x4_t pk;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float a = broken ? __builtin_nanf("") : acc[2 * q];
    const float b = broken ? __builtin_nanf("") : acc[2 * q + 1];
    pk[q] = uint32_t(f32_to_bf16(a)) | (uint32_t(f32_to_bf16(b)) << 16);
  }
  *reinterpret_cast<u32x4_t*>(out + int64_t(tok) * d + 8 * c8) = pk;
}

}  // namespace

int launch_combine(const CombineArgs& a, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const unsigned blocks = unsigned((a.d + kCombineCols - 1) / kCombineCols);
  launch_kernel(combine_kernel, dim3(unsigned(a.t), blocks), dim3(256), s, a.o, a.m_total, a.d, a.k, a.topk,
                a.weights, a.ne, a.seg_offsets, a.row_index, a.out);
  return int(hipGetLastError());
}

}  // namespace qmm
