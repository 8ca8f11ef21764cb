// Decode GEMV y = Ŵ·x for 4-bit weights on gfx950, dense and grouped (one
// launch over all routed experts).
//
// Work split.  A workgroup owns a block of `rows` consecutive output rows and
// the whole of D.  D is cut into slices of 512 codes; wave w of the group
// handles slices w, w + nwaves, ...  Inside a wave, lane l works on row
// (l / 16) of the current row quad and on the 32-code chunk (l % 16) of the
// slice, so each 16-byte code load is one chunk of one row and a wave load
// instruction reads 4 rows × 256 contiguous bytes.  The lane keeps its 32
// activations in registers for the whole slice (they are the same for every
// row), so activations are read once per workgroup and slice.
//
// Per chunk the dot product runs on 2-wide bf16 dot instructions against
// (128 + q) built by OR-ing each nibble pair into the bf16 constant 128.0 (the
// pre-scaling idea of "Step 4: Pre-scaling Nibble Extraction", LLM Decode /
// Prefill 优化案例（Metal）: fold the extraction into one masked OR instead of
// separate shift, mask and subtract), then the group's scale and bias are
// applied once per chunk:
//   Σ x·(s·q + b) = s·(Σ x·(128+q) − 128·Σx) + b·Σx,
// with Σx of the chunk computed once per slice.  MXFP4 chunks are exactly one
// 32-code group: the gfx950 FP4 -> bf16 pair conversion feeds the same dot
// and 2^(E−127) is applied to the chunk sum.
//
// Reduction: a lane accumulates its chunks' partial sums over the slices of
// its wave in registers, the 16 lanes of a row are summed with DPP in a fixed
// order, and the waves are summed in wave order through LDS.  No atomics:
// results are bitwise reproducible.
#include <hip/hip_runtime.h>

#include <stdlib.h>

#include "qmm_device.h"
#include "qmm_internal.h"

namespace qmm {
namespace {

constexpr int kSlice = 512;      // codes per slice (16 lanes × 32 codes)
constexpr int kMaxWaves = 16;

// One pass covers 4·RQ rows: every lane issues the loads of all RQ row quads
// of a slice before it consumes any of them, so a wave keeps RQ 16-byte code
// loads (plus their metadata) in flight.  Addresses of rows past the end are
// clamped to the last row and their results masked, so no load sits behind a
// branch.
template <int FMT, int RQ, bool GROUPED>
__global__ __launch_bounds__(1024) void gemv_kernel(
    const uint8_t* __restrict__ base, int64_t expert_stride, int n_experts,
    int64_t codes_off, int64_t meta_off, int n, int d,
    const uint16_t* __restrict__ x, int64_t t_x, const int32_t* __restrict__ row_index,
    const int32_t* __restrict__ seg_expert, const int32_t* __restrict__ seg_offsets, int m_total,
    uint16_t* __restrict__ y, int rows) {
  __shared__ float red[kMaxWaves][4 * RQ];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  const int rsub = lane >> 4;  // row within the quad
  const int c = lane & 15;     // chunk within the slice
  const int nslices = (d + kSlice - 1) / kSlice;
  const int row0 = blockIdx.x * rows;
  const int row_end = min(row0 + rows, n);
  const int64_t row_bytes = d / 2;
  const int groups = FMT == QMM_AFFINE4_G64 ? d / 64 : d / 32;

  // Segment bookkeeping (grouped): this workgroup serves every grouped row of
  // segment blockIdx.y, one after the other.
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
  const uint8_t* codes = blob + codes_off;
  const uint8_t* meta = blob + meta_off;

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

    for (int p0 = row0; p0 < row_end; p0 += 4 * RQ) {
      float acc[RQ];
#pragma unroll
      for (int q = 0; q < RQ; ++q) acc[q] = 0.f;

      for (int s = wave; s < nslices; s += nwaves) {
        const int kc_raw = s * kSlice + c * 32;  // first code of this lane's chunk
        const bool kvalid = kc_raw < d;
        const int kc = kvalid ? kc_raw : d - 32;
        const int g = FMT == QMM_AFFINE4_G64 ? kc / 64 : kc / 32;

        const uint16_t* px = xr + kc;
        const u32x4_t v0 = load16(px), v1 = load16(px + 8), v2 = load16(px + 16), v3 = load16(px + 24);
        u32x4_t w[RQ];
        uint32_t m[RQ];
#pragma unroll
        for (int q = 0; q < RQ; ++q) {
          const int r = min(p0 + 4 * q + rsub, row_end - 1);
          w[q] = load16(codes + int64_t(r) * row_bytes + kc / 2);
          if (FMT == QMM_AFFINE4_G64)
            m[q] = reinterpret_cast<const uint32_t*>(meta)[int64_t(r) * groups + g];
          else
            m[q] = meta[int64_t(r) * groups + g];
        }
        uint32_t xp[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          xp[i] = v0[i];
          xp[4 + i] = v1[i];
          xp[8 + i] = v2[i];
          xp[12 + i] = v3[i];
        }
        float xsum = 0.f;
        if (FMT == QMM_AFFINE4_G64) {
#pragma unroll
          for (int i = 0; i < 16; ++i) xsum += bf16_lo(xp[i]) + bf16_hi(xp[i]);
        }
#pragma unroll
        for (int q = 0; q < RQ; ++q) {
          float p;
          if (FMT == QMM_AFFINE4_G64) {
            const float dot = affine_dot32(w[q], xp);
            const float sc = bf16_lo(m[q]), bi = bf16_hi(m[q]);
            p = __builtin_fmaf(sc, __builtin_fmaf(-128.f, xsum, dot), bi * xsum);
          } else {
            p = __builtin_ldexpf(mxfp4_dot32(w[q], xp), int(m[q]) - 127);
          }
          acc[q] += kvalid ? p : 0.f;
        }
      }

      // lanes of a row hold partial sums of their chunks: reduce, park per wave
#pragma unroll
      for (int q = 0; q < RQ; ++q) {
        const float v = sum16(acc[q]);
        if (c == 0) red[wave][4 * q + rsub] = v;
      }
      __syncthreads();
      const int nw = min(nwaves, nslices);
      const int rows_here = min(4 * RQ, row_end - p0);
      for (int i = threadIdx.x; i < rows_here; i += blockDim.x) {
        float sum = 0.f;
        for (int w2 = 0; w2 < nw; ++w2) sum += red[w2][i];
        if (GROUPED && bad_row) sum = __builtin_nanf("");
        yr[p0 + i] = f32_to_bf16(sum);
      }
      __syncthreads();
    }
  }
}

template <int FMT, bool GROUPED>
void launch_one(const GemvArgs& a, const Layout& l, int rows, int rq, dim3 grid, int threads,
                hipStream_t s) {
#define QMM_GEMV_LAUNCH(R)                                                                  \
  hipLaunchKernelGGL((gemv_kernel<FMT, R, GROUPED>), grid, dim3(threads), 0, s, a.packed,   \
                     a.expert_stride, a.n_experts, l.codes_offset, l.meta_offset, a.n, a.d, \
                     a.x, a.t_x, a.row_index, a.seg_expert, a.seg_offsets, a.m_total, a.y, rows)
  if (rq <= 2) {
    QMM_GEMV_LAUNCH(2);
  } else if (rq <= 4) {
    QMM_GEMV_LAUNCH(4);
  } else {
    QMM_GEMV_LAUNCH(8);  // more rows run as several passes of 32
  }
#undef QMM_GEMV_LAUNCH
}

int env_int(const char* name, int dflt) {
  const char* v = getenv(name);
  return v && *v ? atoi(v) : dflt;
}

}  // namespace

int launch_gemv(const GemvArgs& a, void* stream) {
  Layout l;
  if (!layout_of(a.f, a.n, a.d, &l)) return int(hipErrorInvalidValue);
  DevInfo info;
  int err = device_info(&info);
  if (err) return err;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int nslices = (a.d + kSlice - 1) / kSlice;
  const int nwaves = nslices < kMaxWaves ? nslices : kMaxWaves;
  const int threads = 64 * nwaves;
  // Rows per workgroup: `per_cu` workgroups per CU across all segments.
  const int nseg = a.n_seg > 0 ? a.n_seg : 1;
  const int per_cu = env_int("QMM_GEMV_WG_PER_CU", 2);
  const int64_t target_wgs = int64_t(info.cus) * (per_cu > 0 ? per_cu : 1);
  int64_t rows = (int64_t(a.n) * nseg + target_wgs - 1) / target_wgs;
  const int env_rows = env_int("QMM_GEMV_ROWS", 0);
  if (env_rows > 0) rows = env_rows;
  if (rows < 1) rows = 1;
  if (rows > 4096) rows = 4096;
  // row quads in flight per pass: just enough to cover the workgroup's rows
  const int rq = int((rows + 3) / 4);
  dim3 grid(unsigned((a.n + rows - 1) / rows), unsigned(nseg));
  if (a.n_seg > 0) {
    if (a.f == QMM_AFFINE4_G64)
      launch_one<QMM_AFFINE4_G64, true>(a, l, int(rows), rq, grid, threads, s);
    else
      launch_one<QMM_MXFP4_G32, true>(a, l, int(rows), rq, grid, threads, s);
  } else {
    if (a.f == QMM_AFFINE4_G64)
      launch_one<QMM_AFFINE4_G64, false>(a, l, int(rows), rq, grid, threads, s);
    else
      launch_one<QMM_MXFP4_G32, false>(a, l, int(rows), rq, grid, threads, s);
  }
  return int(hipGetLastError());
}

}  // namespace qmm
