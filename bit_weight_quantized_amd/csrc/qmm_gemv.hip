// Decode GEMV y = Ŵ·x for 4-bit weights on gfx950, dense and grouped (one
// launch over all routed experts).
//
// Work split.  A wave owns one quad of 4 consecutive output rows across the
// whole reduction axis; lane l works on row (l / 16) of the quad and on the
// 32-code chunk (l % 16) of the current 512-code slab.  With the K-slabbed
// packed layout the quad's 4 rows of one slab are 1 KiB contiguous, so each
// wave load instruction is one contiguous 1 KiB, and since every wave walks
// the slabs in the same order the whole GPU sweeps the weights front to back
// like a streaming copy.  No work is split across waves: no barrier after the
// prologue, no cross-wave reduction.  Each lane keeps a ring of kPF slabs of
// code and metadata loads in flight.
//
// Activations.  The workgroup stages the activation row and the sums of its
// 32-code chunks in LDS once (D <= 16384); each lane reads its chunk of a slab
// when it consumes it.  Larger D reads them from global memory instead.
//
// Arithmetic.  Per chunk the dot product runs on 2-wide bf16 dot instructions
// against (128 + q), built by OR-ing each nibble pair into the bf16 constant
// 128.0 with one masked OR (the pre-scaling idea of "Step 4: Pre-scaling Nibble
// Extraction", LLM Decode / Prefill 优化案例（Metal）: fold extraction into one
// instruction instead of separate shift, mask and subtract); the group's scale
// and bias are then applied once per chunk:
//   Σ x·(s·q + b) = s·(Σ x·(128+q) − 128·Σx) + b·Σx.
// MXFP4 chunks are exactly one 32-code group: the gfx950 FP4 -> bf16 pair
// conversion feeds the same dot and 2^(E−127) is applied to the chunk sum.
//
// Reduction: each lane accumulates its chunks over all slabs in registers,
// then the 16 lanes of a row are summed with DPP in a fixed order.  No
// atomics: results are bitwise reproducible.
#include <hip/hip_runtime.h>

#include <stdlib.h>

#include "qmm_device.h"
#include "qmm_internal.h"
#include "qmm_launch.h"

namespace qmm {
namespace {

constexpr int kPF = 4;          // slabs in flight per lane
constexpr int kXldsMaxD = 16384;
// Activations sit in LDS as 32-code chunks of 64 bytes at a stride of 80
// bytes: the 8 lanes of one LDS access phase then read 16-byte pieces that
// start 20 banks apart, covering all 32 banks once (a 64-byte stride would put
// every other lane on the same 16 banks).
constexpr int kXChunkStride = 40;  // in bf16

template <int FMT>
struct SlabLoad {
  u32x4_t w;   // 32 codes
  uint32_t m;  // their group metadata
};

// The 32 activations of one chunk as bf16 pairs, and their sum (affine only):
// from LDS at byte offset `xa` / `ca` (staged), or from global memory.
template <int FMT, bool XLDS>
__device__ __forceinline__ void read_x(const uint8_t* smem, uint32_t xa, uint32_t ca,
                                       const uint16_t* xg, uint32_t* xp, float& xsum) {
  u32x4_t v0, v1, v2, v3;
  if (XLDS) {
    const uint8_t* p = smem + xa;
    v0 = *reinterpret_cast<const u32x4_t*>(p);
    v1 = *reinterpret_cast<const u32x4_t*>(p + 16);
    v2 = *reinterpret_cast<const u32x4_t*>(p + 32);
    v3 = *reinterpret_cast<const u32x4_t*>(p + 48);
  } else {
    v0 = load16(xg);
    v1 = load16(xg + 8);
    v2 = load16(xg + 16);
    v3 = load16(xg + 24);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    xp[i] = v0[i];
    xp[4 + i] = v1[i];
    xp[8 + i] = v2[i];
    xp[12 + i] = v3[i];
  }
  if (FMT == QMM_AFFINE4_G64) {
    if (XLDS) {
      xsum = *reinterpret_cast<const float*>(smem + ca);
    } else {
      float a = 0.f, b = 0.f;
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        a = dot2_bf16(xp[i], 0x3F803F80u, a);      // (1.0, 1.0)
        b = dot2_bf16(xp[i + 1], 0x3F803F80u, b);
      }
      xsum = a + b;
    }
  }
}

template <int FMT>
__device__ __forceinline__ float chunk_partial(const SlabLoad<FMT>& b, const uint32_t* xp,
                                               float xsum) {
  if (FMT == QMM_AFFINE4_G64) {
    const float dot = affine_dot32(b.w, xp);
    const float sc = bf16_lo(b.m), bi = bf16_hi(b.m);
    return __builtin_fmaf(sc, __builtin_fmaf(-128.f, xsum, dot), bi * xsum);
  }
  return __builtin_ldexpf(mxfp4_dot32(b.w, xp), int(b.m) - 127);
}

template <int FMT, bool XLDS, bool GROUPED>
__global__ __launch_bounds__(256) void gemv_kernel(
    const uint8_t* __restrict__ base, int64_t expert_stride, int n_experts,
    int64_t codes_off, int64_t meta_off, uint32_t codes_bytes, uint32_t meta_bytes, int n, int d,
    const uint16_t* __restrict__ x, int64_t t_x, const int32_t* __restrict__ row_index,
    const int32_t* __restrict__ seg_expert, const int32_t* __restrict__ seg_offsets, int m_total,
    uint16_t* __restrict__ y) {
  // LDS: activation chunks (80-byte stride) for whole slabs, then chunk sums
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const Slabs L{n, d, FMT};
  const int nslabs = L.count();
  const int nchunks = d / 32;
  const uint32_t csum_base = uint32_t(nslabs) * 16u * (2 * kXChunkStride);
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);
  float* csum = reinterpret_cast<float*>(smem + csum_base);

  const int lane = threadIdx.x & 63;
  const int rsub = lane >> 4;
  const int c = lane & 15;
  const int wpg = blockDim.x >> 6;
  const int wrow0 = (blockIdx.x * wpg + (threadIdx.x >> 6)) * 4;   // this wave's quad
  const int row = wrow0 + rsub;
  const int slast = nslabs - 1;
  const bool partial_last = L.width(slast) < kSlabCodes;
  const bool lane_in_last = 32 * c < L.width(slast);

  int r_begin = 0, r_end = 1;
  const uint8_t* blob = base;
  bool bad_expert = false;
  if (GROUPED) {
    const int s = blockIdx.y;
    r_begin = min(max(seg_offsets[s], 0), m_total);
    r_end = min(max(seg_offsets[s + 1], r_begin), m_total);
    const int e = seg_expert[s];
    bad_expert = e < 0 || e >= n_experts;
    blob = base + (bad_expert ? 0 : int64_t(e) * expert_stride);
  }
  // Whole code / metadata sections.  Rows >= n only occur in the last quad;
  // their loads are pointed at row n - 1 and their results never stored.
  const __amdgpu_buffer_rsrc_t cr = make_rsrc(blob + codes_off, codes_bytes);
  const __amdgpu_buffer_rsrc_t mr = make_rsrc(blob + meta_off, meta_bytes);
  const int lrow = min(row, n - 1);
  // this lane's chunk in full slab s sits at base + s * step (K-slabbed layout)
  const uint32_t mslab = FMT == QMM_AFFINE4_G64 ? 32u : 16u;   // metadata bytes per row per full slab
  const uint32_t mlane = FMT == QMM_AFFINE4_G64 ? 4u * uint32_t(c / 2) : uint32_t(c);
  const uint32_t co0 = uint32_t(lrow) * (kSlabCodes / 2) + uint32_t(16 * c);
  const uint32_t mo0 = uint32_t(lrow) * mslab + mlane;
  const uint32_t cstep = uint32_t(n) * (kSlabCodes / 2), mstep = uint32_t(n) * mslab;
  // the last slab may be narrower; its rows are packed at its own width
  const uint32_t co_last = uint32_t(L.codes(slast, lrow)) + uint32_t(16 * c);
  const uint32_t mo_last = uint32_t(L.meta(slast, lrow)) + mlane;

  for (int gr = r_begin; gr < r_end; ++gr) {
    const uint16_t* xr = x;
    uint16_t* yr = y;
    bool bad_row = false;
    if (GROUPED) {
      const int src = row_index[gr];
      bad_row = bad_expert || src < 0 || src >= t_x;
      xr = x + (bad_row ? 0 : int64_t(src) * d);
      yr = y + int64_t(gr) * n;
    }
    auto issue = [&](SlabLoad<FMT>& b, int s) {
      const bool last = partial_last && s == slast;
      const uint32_t co = last ? co_last : co0 + uint32_t(s) * cstep;
      const uint32_t mo = last ? mo_last : mo0 + uint32_t(s) * mstep;
      b.w = buf_load16(cr, co);
      b.m = FMT == QMM_AFFINE4_G64 ? buf_load4(mr, mo) : buf_load1(mr, mo);
    };
    // start the weight stream before the activation staging
    SlabLoad<FMT> ring[kPF];
#pragma unroll
    for (int j = 0; j < kPF; ++j)
      if (j < nslabs) issue(ring[j], j);
    if (XLDS) {
      __syncthreads();  // the previous row's readers are done with xs
      for (int i = threadIdx.x; i < d / 8; i += blockDim.x)
        *reinterpret_cast<u32x4_t*>(xs + (i >> 2) * kXChunkStride + 8 * (i & 3)) = load16(xr + 8 * i);
      __syncthreads();
      if (FMT == QMM_AFFINE4_G64) {
        for (int i = threadIdx.x; i < nchunks; i += blockDim.x) {
          const uint16_t* p = xs + i * kXChunkStride;
          float a = 0.f, b = 0.f;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const u32x4_t v = *reinterpret_cast<const u32x4_t*>(p + 8 * j);
            a = dot2_bf16(v[0], 0x3F803F80u, a);
            b = dot2_bf16(v[1], 0x3F803F80u, b);
            a = dot2_bf16(v[2], 0x3F803F80u, a);
            b = dot2_bf16(v[3], 0x3F803F80u, b);
          }
          csum[i] = a + b;
        }
        __syncthreads();
      }
    }

    // running activation offsets of this lane's chunk (LDS bytes / global elements)
    uint32_t xa = uint32_t(c) * (2 * kXChunkStride), ca = csum_base + 4u * uint32_t(c);
    const uint16_t* xg = xr + 32 * c;
    float acc = 0.f;
    for (int s0 = 0; s0 < nslabs; s0 += kPF) {
#pragma unroll
      for (int j = 0; j < kPF; ++j) {
        const int s = s0 + j;
        if (s < nslabs) {
          uint32_t xp[16];
          float xsum = 0.f;
          // the chunk may lie past D in a partial last slab: keep global reads in range
          read_x<FMT, XLDS>(smem, xa, ca, XLDS ? xg : (lane_in_last || s != slast ? xg : xr), xp, xsum);
          const float p = chunk_partial<FMT>(ring[j], xp, xsum);
          acc += (!partial_last || s != slast || lane_in_last) ? p : 0.f;
          if (s + kPF < nslabs) issue(ring[j], s + kPF);
          xa += 16u * (2 * kXChunkStride);
          ca += 64u;
          xg += kSlabCodes;
        }
      }
    }
    const float v = sum16(acc);
    if (c == 0 && row < n) yr[row] = f32_to_bf16((GROUPED && bad_row) ? __builtin_nanf("") : v);
  }
}

int env_int(const char* name, int dflt) {
  const char* v = getenv(name);
  return v && *v ? atoi(v) : dflt;
}

template <int FMT, bool GROUPED>
void launch_fmt(const GemvArgs& a, const Layout& l, dim3 grid, int threads, hipStream_t s) {
  const uint32_t codes_bytes = uint32_t(int64_t(a.n) * (a.d / 2));
  const uint32_t meta_bytes = uint32_t(l.meta_bytes);
  if (a.d <= kXldsMaxD) {
    const size_t slabs = size_t((a.d + kSlabCodes - 1) / kSlabCodes);
    const size_t lds = slabs * 16 * (2 * kXChunkStride + 4);
    launch_kernel_lds((gemv_kernel<FMT, true, GROUPED>), grid, dim3(threads), lds, s, a.packed,
                      a.expert_stride, a.n_experts, l.codes_offset, l.meta_offset, codes_bytes,
                      meta_bytes, a.n, a.d, a.x, a.t_x, a.row_index, a.seg_expert, a.seg_offsets,
                      a.m_total, a.y);
  } else {
    launch_kernel_lds((gemv_kernel<FMT, false, GROUPED>), grid, dim3(threads), 0, s, a.packed,
                      a.expert_stride, a.n_experts, l.codes_offset, l.meta_offset, codes_bytes,
                      meta_bytes, a.n, a.d, a.x, a.t_x, a.row_index, a.seg_expert, a.seg_offsets,
                      a.m_total, a.y);
  }
}

}  // namespace

int launch_gemv(const GemvArgs& a, void* stream) {
  Layout l;
  if (!layout_of(a.f, a.n, a.d, &l)) return int(hipErrorInvalidValue);
  // 32-bit buffer offsets: one blob's codes must stay under 2 GiB
  if (int64_t(a.n) * (a.d / 2) >= (int64_t(1) << 31)) return int(hipErrorInvalidValue);
  hipStream_t s = static_cast<hipStream_t>(stream);
  int wpg = env_int("QMM_GEMV_WPG", 4);   // waves (row quads) per workgroup
  if (wpg < 1) wpg = 1;
  if (wpg > 4) wpg = 4;
  const int nseg = a.n_seg > 0 ? a.n_seg : 1;
  const int wrows = 4 * wpg;
  dim3 grid(unsigned((a.n + wrows - 1) / wrows), unsigned(nseg));
  if (a.n_seg > 0) {
    if (a.f == QMM_AFFINE4_G64)
      launch_fmt<QMM_AFFINE4_G64, true>(a, l, grid, 64 * wpg, s);
    else
      launch_fmt<QMM_MXFP4_G32, true>(a, l, grid, 64 * wpg, s);
  } else {
    if (a.f == QMM_AFFINE4_G64)
      launch_fmt<QMM_AFFINE4_G64, false>(a, l, grid, 64 * wpg, s);
    else
      launch_fmt<QMM_MXFP4_G32, false>(a, l, grid, 64 * wpg, s);
  }
  return int(hipGetLastError());
}

}  // namespace qmm
