// Prefill GEMM and routed-expert grouped GEMM on gfx950 MFMA.
//
// Y = X·Ŵᵀ is the one dense contraction of the path, so it runs on bf16 MFMA
// with fp32 accumulation.  Weights stay 4-bit in HBM: each wave streams the
// packed codes of its own output columns straight from global memory into
// registers, dequantises them there into bf16 MFMA B operands, and never
// writes dequantised weights back to memory (materialising them would move
// four times the bytes).  Activation tiles are shared by the four waves of a
// workgroup through LDS.
//
// k order inside a K step.  An MFMA sums over its k positions in any order,
// so the k index a lane supplies only has to agree between its A and B
// operands.  Lane group g (lanes with the same l / 32, or l / 16 for 16x16)
// holds the contiguous 32-code chunk g of the K step, i.e. one 16-byte load of
// codes, and MFMA j of the step consumes word j of that chunk.  The A operand
// of the same lane is read from LDS at the matching k offset (32g + 8j).
//
// Dense kernel: workgroup tile WM×256, wave w owns columns [64w, 64w + 64)
// and all WM rows, v_mfma_f32_32x32x16_bf16, K step 64 (one affine group).
// Grouped kernel: one workgroup per (segment, 256-column tile), rows of the
// segment gathered through row_index in blocks of 64, 16x16x32 MFMA so short
// segments waste little, K step 128.  Each expert's weight tile is read once
// per 64 routed rows.
#include <hip/hip_runtime.h>

#include "qmm_device.h"
#include "qmm_internal.h"
#include "qmm_launch.h"

namespace qmm {
namespace {

// B operand of K-step chunk word j for one lane.
template <int FMT>
__device__ __forceinline__ void dequant_chunk(const u32x4_t w, uint32_t m, u32x4_t out[4]) {
  if (FMT == QMM_AFFINE4_G64) {
    const float s = bf16_lo(m), b = bf16_hi(m);
#pragma unroll
    for (int j = 0; j < 4; ++j) out[j] = affine_word_to_bf16x8(w[j], s, b);
  } else {
    const float sc = e8m0_scale(m);
#pragma unroll
    for (int j = 0; j < 4; ++j) out[j] = mxfp4_word_to_bf16x8(w[j], sc);
  }
}

// Codes [k, k + 32) of weight row `col` (one 16-byte chunk) and the metadata
// of their group, from the K-slabbed layout (qmm_internal.h).
template <int FMT>
__device__ __forceinline__ void load_chunk(const uint8_t* codes, const uint8_t* meta,
                                           const Slabs& L, int64_t col, int k, u32x4_t& w,
                                           uint32_t& m) {
  w = load16(codes + L.code_byte(col, k));
  if (FMT == QMM_AFFINE4_G64)
    m = *reinterpret_cast<const uint32_t*>(meta + L.meta_byte(col, k));
  else
    m = meta[L.meta_byte(col, k)];
}

// ---------------------------------------------------------------------------
// Dense GEMM
// ---------------------------------------------------------------------------
constexpr int kXs = 72;  // LDS row stride in bf16 for a 64-wide K step (16-byte pad)

template <int FMT, int WM>
__global__ __launch_bounds__(256) void gemm_kernel(const uint8_t* __restrict__ codes,
                                                   const uint8_t* __restrict__ meta, int t, int n,
                                                   int d, const uint16_t* __restrict__ x,
                                                   uint16_t* __restrict__ y, int tiles_m,
                                                   int tiles_n) {
  constexpr int RB = WM / 32;
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][WM * kXs];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col_l = lane & 31, g = lane >> 5;

  // XCD-aware tile order: consecutive workgroups are dealt round-robin to the
  // 8 XCDs; give each XCD a contiguous run of tiles, N fastest, so the
  // workgroups of one XCD share an activation strip in that XCD's L2.
  const int tiles = tiles_m * tiles_n;
  int tile = blockIdx.x;
  if ((tiles & 7) == 0) tile = (blockIdx.x & 7) * (tiles >> 3) + (blockIdx.x >> 3);
  const int tm = tile / tiles_n, tn = tile % tiles_n;
  const int m0 = tm * WM, n0 = tn * 256;

  const Slabs L{n, d, FMT};
  const int nk = (d + 63) / 64;

  // this lane's two weight columns
  int64_t col[2];
  bool col_ok[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    col[cb] = n0 + 64 * wave + 32 * cb + col_l;
    col_ok[cb] = col[cb] < n;
  }

  // activation tile loader: thread -> row (tid / 8) + 32 i, 16-byte slot tid % 8
  const int xr = tid >> 3, xslot = tid & 7;
  u32x4_t xreg[RB];
  auto load_x = [&](int k0) {
    const int k = k0 + 8 * xslot;
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const int row = m0 + xr + 32 * i;
      xreg[i] = (row < t && k < d) ? load16(x + int64_t(row) * d + k) : u32x4_t{0, 0, 0, 0};
    }
  };
  auto store_x = [&](int buf) {
#pragma unroll
    for (int i = 0; i < RB; ++i)
      *reinterpret_cast<u32x4_t*>(&xs[buf][(xr + 32 * i) * kXs + 8 * xslot]) = xreg[i];
  };

  u32x4_t wreg[2];
  uint32_t mreg[2];
  auto load_w = [&](int k0) {
    const int k = k0 + 32 * g;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      if (col_ok[cb] && k < d) {
        load_chunk<FMT>(codes, meta, L, col[cb], k, wreg[cb], mreg[cb]);
      } else {
        wreg[cb] = u32x4_t{0, 0, 0, 0};
        mreg[cb] = 0;
      }
    }
  };

  f32x16_t acc[RB][2];
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][cb][r] = 0.f;

  load_x(0);
  load_w(0);
  store_x(0);

  for (int ks = 0; ks < nk; ++ks) {
    const int buf = ks & 1;
    const int k0 = ks * 64;
    u32x4_t bfrag[2][4];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      dequant_chunk<FMT>(wreg[cb], mreg[cb], bfrag[cb]);
      if (!(col_ok[cb] && k0 + 32 * g < d))
#pragma unroll
        for (int j = 0; j < 4; ++j) bfrag[cb][j] = u32x4_t{0, 0, 0, 0};
    }
    if (ks + 1 < nk) {
      load_x(k0 + 64);
      load_w(k0 + 64);
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        const u32x4_t a = *reinterpret_cast<const u32x4_t*>(&xs[buf][(32 * i + col_l) * kXs + 32 * g + 8 * j]);
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
          acc[i][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, bfrag[cb][j]),
              acc[i][cb], 0, 0, 0);
      }
    }
    if (ks + 1 < nk) store_x(buf ^ 1);
  }

  // epilogue: lane holds column col_l of each 32x32 block, rows 8(r/4) + 4g + r%4
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      if (!col_ok[cb]) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + 32 * i + 8 * (r >> 2) + 4 * g + (r & 3);
        if (row < t) y[int64_t(row) * n + col[cb]] = f32_to_bf16(acc[i][cb][r]);
      }
    }
}

// ---------------------------------------------------------------------------
// Grouped GEMM (routed experts)
// ---------------------------------------------------------------------------
constexpr int kGBM = 64;    // routed rows per pass
constexpr int kGXs = 136;   // LDS row stride in bf16 for a 128-wide K step

template <int FMT>
__global__ __launch_bounds__(256) void grouped_gemm_kernel(
    const uint8_t* __restrict__ base, int64_t expert_stride, int n_experts, int64_t codes_off,
    int64_t meta_off, int n, int d, const uint16_t* __restrict__ x, int64_t t_x,
    const int32_t* __restrict__ row_index, const int32_t* __restrict__ seg_expert,
    const int32_t* __restrict__ seg_offsets, int m_total, uint16_t* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][kGBM * kGXs];
  __shared__ int32_t src_row[kGBM];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col_l = lane & 15, g = lane >> 4;
  const int s = blockIdx.y;
  const int n0 = blockIdx.x * 256;

  const int r_begin = min(max(seg_offsets[s], 0), m_total);
  const int r_end = min(max(seg_offsets[s + 1], r_begin), m_total);
  if (r_begin >= r_end) return;
  const int e = seg_expert[s];
  const bool bad_expert = e < 0 || e >= n_experts;
  const uint8_t* blob = base + (bad_expert ? 0 : int64_t(e) * expert_stride);
  const uint8_t* codes = blob + codes_off;
  const uint8_t* meta = blob + meta_off;

  const Slabs L{n, d, FMT};
  const int nk = (d + 127) / 128;

  int64_t col[4];
  bool col_ok[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
    col[cb] = n0 + 64 * wave + 16 * cb + col_l;
    col_ok[cb] = col[cb] < n;
  }

  const int xr = tid >> 2, xq = tid & 3;  // activation loader: row tid/4, slots 4xq..4xq+3

  for (int mb = r_begin; mb < r_end; mb += kGBM) {
    const int nrows = min(kGBM, r_end - mb);
    const int nrb = (nrows + 15) >> 4;
    if (tid < kGBM) {
      int src = -1;
      if (tid < nrows) {
        src = row_index[mb + tid];
        if (bad_expert || src < 0 || src >= t_x) src = -2;
      }
      src_row[tid] = src;
    }
    __syncthreads();
    const int my_src = src_row[xr];

    u32x4_t xreg[4];
    auto load_x = [&](int k0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int k = k0 + 8 * (4 * xq + i);
        xreg[i] = (my_src >= 0 && k < d) ? load16(x + int64_t(my_src) * d + k) : u32x4_t{0, 0, 0, 0};
      }
    };
    auto store_x = [&](int buf) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<u32x4_t*>(&xs[buf][xr * kGXs + 8 * (4 * xq + i)]) = xreg[i];
    };
    u32x4_t wreg[4];
    uint32_t mreg[4];
    auto load_w = [&](int k0) {
      const int k = k0 + 32 * g;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        if (col_ok[cb] && k < d) {
          load_chunk<FMT>(codes, meta, L, col[cb], k, wreg[cb], mreg[cb]);
        } else {
          wreg[cb] = u32x4_t{0, 0, 0, 0};
          mreg[cb] = 0;
        }
      }
    };

    f32x4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) acc[i][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    load_x(0);
    load_w(0);
    store_x(0);
    for (int ks = 0; ks < nk; ++ks) {
      const int buf = ks & 1;
      const int k0 = ks * 128;
      u32x4_t bfrag[4][4];
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        dequant_chunk<FMT>(wreg[cb], mreg[cb], bfrag[cb]);
        if (!(col_ok[cb] && k0 + 32 * g < d))
#pragma unroll
          for (int j = 0; j < 4; ++j) bfrag[cb][j] = u32x4_t{0, 0, 0, 0};
      }
      if (ks + 1 < nk) {
        load_x(k0 + 128);
        load_w(k0 + 128);
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (i < nrb) {
            const u32x4_t a = *reinterpret_cast<const u32x4_t*>(&xs[buf][(16 * i + col_l) * kGXs + 32 * g + 8 * j]);
#pragma unroll
            for (int cb = 0; cb < 4; ++cb)
              acc[i][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  __builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, bfrag[cb][j]),
                  acc[i][cb], 0, 0, 0);
          }
        }
      }
      if (ks + 1 < nk) store_x(buf ^ 1);
    }

    // epilogue: lane holds column col_l, rows 4g + r of each 16x16 block
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i >= nrb) continue;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        if (!col_ok[cb]) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int lr = 16 * i + 4 * g + r;
          if (lr < nrows) {
            const float v = src_row[lr] == -2 ? __builtin_nanf("") : acc[i][cb][r];
            y[int64_t(mb + lr) * n + col[cb]] = f32_to_bf16(v);
          }
        }
      }
    }
    __syncthreads();  // src_row and xs are reused by the next pass
  }
}

}  // namespace

int launch_gemm(const GemmArgs& a, void* stream) {
  Layout l;
  if (!layout_of(a.f, a.n, a.d, &l)) return int(hipErrorInvalidValue);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint8_t* codes = a.packed + l.codes_offset;
  const uint8_t* meta = a.packed + l.meta_offset;
  const int tiles_n = (a.n + 255) / 256;
  // 256-row tiles for tall X, 128-row tiles otherwise
  if (a.t > 128) {
    const int tiles_m = (a.t + 255) / 256;
    dim3 grid(unsigned(tiles_m * tiles_n));
    if (a.f == QMM_AFFINE4_G64)
      launch_kernel((gemm_kernel<QMM_AFFINE4_G64, 256>), grid, dim3(256), s, codes, meta,
                         a.t, a.n, a.d, a.x, a.y, tiles_m, tiles_n);
    else
      launch_kernel((gemm_kernel<QMM_MXFP4_G32, 256>), grid, dim3(256), s, codes, meta,
                         a.t, a.n, a.d, a.x, a.y, tiles_m, tiles_n);
  } else {
    const int tiles_m = (a.t + 127) / 128;
    dim3 grid(unsigned(tiles_m * tiles_n));
    if (a.f == QMM_AFFINE4_G64)
      launch_kernel((gemm_kernel<QMM_AFFINE4_G64, 128>), grid, dim3(256), s, codes, meta,
                         a.t, a.n, a.d, a.x, a.y, tiles_m, tiles_n);
    else
      launch_kernel((gemm_kernel<QMM_MXFP4_G32, 128>), grid, dim3(256), s, codes, meta,
                         a.t, a.n, a.d, a.x, a.y, tiles_m, tiles_n);
  }
  return int(hipGetLastError());
}

int launch_grouped_gemm(const GemmArgs& a, void* stream) {
  Layout l;
  if (!layout_of(a.f, a.n, a.d, &l)) return int(hipErrorInvalidValue);
  hipStream_t s = static_cast<hipStream_t>(stream);
  dim3 grid(unsigned((a.n + 255) / 256), unsigned(a.n_seg));
  if (a.f == QMM_AFFINE4_G64)
    launch_kernel(grouped_gemm_kernel<QMM_AFFINE4_G64>, grid, dim3(256), s, a.packed,
                       a.expert_stride, a.n_experts, l.codes_offset, l.meta_offset, a.n, a.d, a.x,
                       a.t_x, a.row_index, a.seg_expert, a.seg_offsets, a.m_total, a.y);
  else
    launch_kernel(grouped_gemm_kernel<QMM_MXFP4_G32>, grid, dim3(256), s, a.packed,
                       a.expert_stride, a.n_experts, l.codes_offset, l.meta_offset, a.n, a.d, a.x,
                       a.t_x, a.row_index, a.seg_expert, a.seg_offsets, a.m_total, a.y);
  return int(hipGetLastError());
}

}  // namespace qmm
