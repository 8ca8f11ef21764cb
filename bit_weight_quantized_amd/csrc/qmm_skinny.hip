// Few-row GEMM: Y = X·Ŵᵀ for 2 <= T <= 64 activation rows (a batch of decode
// tokens), the same product as the prefill GEMM ("Kapitsa 源码拆解 02：权重、
// 矩阵与 Metal", section "矩阵乘法中数据和参数") at a size where it is bound by
// the weight stream, like the decode GEMV, yet every weight serves T rows.
//
// A 256-column tile of the output has only one column strip of weights to
// stream, so tiling the output alone leaves most of the chip idle (a 13824-row
// matrix gives 54 tiles).  The work is split along K instead: one workgroup per
// (256-column tile, 512-code slab of d), which for the decode matrix is 540
// workgroups.  Each workgroup issues the whole slab of its columns' codes
// (64 KiB) and their group metadata at once, stages the T activation rows of the
// slab in LDS, dequantises every weight once into bf16 MFMA B operands and
// runs v_mfma_f32_16x16x32_bf16 over the row blocks (rows past T are zeros).
// Its fp32 partial sums go to the caller's workspace, one [T][N] plane per
// slab; a second kernel adds the planes in slab order and rounds once to bf16,
// so the summation order is fixed.  The k order inside a 128-code step is the
// grouped GEMM's: lane group g holds the step's 32-code chunk g, and MFMA j
// takes word j of it against the activations at the same k.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <type_traits>

#include "qmm_device.h"
#include "qmm_internal.h"
#include "qmm_launch.h"
#include "qmm_skinny.h"

namespace qmm {
namespace {

constexpr uint32_t kOOB = 0x80000000u;   // OR-ed into a buffer offset: past every range
// LDS activation slab: row r holds the slab's 512 codes (1 KiB) with 16-byte
// chunk c stored at position c ^ (r & 15), so the 16 rows of one MFMA operand
// read (same chunk) fall in 16 different bank groups
__device__ __forceinline__ int xs_at(int r, int c) { return r * kSlabCodes + ((c ^ (r & 15)) << 3); }
// After the activation slab (affine weights): a block of zeros that half the
// lanes read instead of activations, then the rows' activation sums per
// 64-code group (fp32, up to 64 rows × 8 groups).
constexpr int kZeroElems = 512;
constexpr int kSkExtraBytes = kZeroElems * 2 + 64 * 8 * 4;

// Affine weights with four row blocks hold the most registers (the exact path
// keeps per-group partial sums beside the accumulators): one workgroup per CU,
// which leaves them the whole register file.
template <int FMT, int NRB>
__global__ __launch_bounds__(256, FMT == QMM_AFFINE4_G64 && NRB == 4 ? 1 : 2) void skinny_kernel(const uint8_t* __restrict__ codes,
                                                        const uint8_t* __restrict__ meta,
                                                        uint32_t codes_bytes, uint32_t meta_bytes,
                                                        int t, int n, int d,
                                                        const uint16_t* __restrict__ x,
                                                        float* __restrict__ ws) {
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col_l = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * 256;
  const int sl = blockIdx.y;
  const Slabs L{n, d, FMT};
  const int w = L.width(sl);           // codes of d in this slab
  const int wcol = n0 + 64 * wave;     // the wave's first column
  const __amdgpu_buffer_rsrc_t crs = make_rsrc(codes, codes_bytes);
  const __amdgpu_buffer_rsrc_t mrs = make_rsrc(meta, meta_bytes);
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(x, uint32_t(t) * uint32_t(d) * 2u);

  // 1. every load of the workgroup issued at once, unconditionally (what must
  //    not be read takes an out-of-range offset and reads zeros):
  //    (a) the activation slab, 16-byte pieces p = tid + 256i: row p / 64,
  //        codes 8(p % 64).. of the slab (zeros past t and past d)
  constexpr int XP = NRB * 4;   // pieces per thread
  u32x4_t xv[XP];
#pragma unroll
  for (int i = 0; i < XP; ++i) {
    const int p = tid + 256 * i, r = p >> 6, kc = (p & 63) * 8;
    xv[i] = buf_load16(xrs, r < t && kc < w ? (uint32_t(r) * uint32_t(d) + uint32_t(sl * kSlabCodes + kc)) * 2u : kOOB);
  }
  //    (b) the wave's codes for the whole slab: column block cb, step s (128
  //        codes), lane (col_l, g) the step's 32-code chunk g; chunks past the
  //        slab's width read zeros, columns past n re-read column n - 1 (never stored)
  u32x4_t wr[4][4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
    const int col = min(wcol + 16 * cb + col_l, n - 1);
    const uint32_t cbase = uint32_t(L.codes(sl, col));
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int kk = 128 * s + 32 * g;
      wr[cb][s] = buf_load16(crs, kk < w ? cbase + uint32_t(kk >> 1) : kOOB);
    }
  }
  //    (c) the slab's group metadata of the wave's column `lane`: affine 8
  //        dwords (scale, bias per 64 codes), MXFP4 4 dwords (E8M0 per 32 codes)
  constexpr int MW = FMT == QMM_AFFINE4_G64 ? 8 : 4;
  uint32_t mv[MW];
  {
    const int col = min(wcol + lane, n - 1);
    const uint32_t mo = uint32_t(L.meta(sl, col));
    const int mrow = L.meta_row(sl);
#pragma unroll
    for (int i = 0; i < MW / 4; ++i) {
      const u32x4_t v = buf_load16(mrs, 16 * i < mrow ? mo + 16u * uint32_t(i) : kOOB);
#pragma unroll
      for (int j = 0; j < 4; ++j) mv[4 * i + j] = v[j];
    }
  }

  // 2. the activations to LDS (issued first, so they are the first to arrive)
#pragma unroll
  for (int i = 0; i < XP; ++i) {
    const int p = tid + 256 * i;
    *reinterpret_cast<u32x4_t*>(&xs[xs_at(p >> 6, p & 63)]) = xv[i];
  }
  __syncthreads();

  f32x4_t acc[NRB][4];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  if constexpr (FMT == QMM_AFFINE4_G64) {
    // 3'. Affine: the codes enter the MFMAs as the exact bf16 values 128 + q
    //     (one v_and_or per pair instead of a dequantisation per weight), one
    //     group per MFMA, and scale and bias are applied per group afterwards
    //     in fp32:  Σ_k x·(s·q + b) = s·Σ_k x·(128 + q) + (b − 128·s)·Σ_k x.
    //     No weight is rounded.  A 128-code step holds two groups, lane group
    //     g's chunk lying in group g / 2; the MFMAs of group h read activations
    //     on the lanes of that half and zeros on the others, so each sums one
    //     group only.
    uint16_t* zero = xs + NRB * 16 * kSlabCodes;
    float* xsum = reinterpret_cast<float*>(zero + kZeroElems);
    if (tid < kZeroElems / 8) *reinterpret_cast<u32x4_t*>(zero + 8 * tid) = u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
    for (int p0 = 0; p0 < NRB * 128; p0 += 256) {   // (row, group) p: its 64 activations summed in order
      const int p = p0 + tid;
      if (p < NRB * 128) {
        const int r = p >> 3, gr = p & 7;
        float sum = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const u32x4_t v = *reinterpret_cast<const u32x4_t*>(&xs[xs_at(r, 8 * gr + c)]);
#pragma unroll
          for (int q = 0; q < 4; ++q) sum = (sum + bf16_lo(v[q])) + bf16_hi(v[q]);
        }
        xsum[r * 8 + gr] = sum;
      }
    }
    __syncthreads();
    const int gh = g >> 1;
    const int zoff = NRB * 16 * kSlabCodes;   // the zero block, as an element offset
    int own[4];   // element offset of word j's activations in row block 0 (step 0)
#pragma unroll
    for (int j = 0; j < 4; ++j) own[j] = col_l * kSlabCodes + (((4 * g + j) ^ col_l) << 3);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (128 * s >= w) break;   // a narrow last slab ends early (uniform)
      float gs[4][2], gc[4][2];   // scale and b − 128·s of groups 2s, 2s + 1 for the lane's column
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const int src = 4 * (16 * cb + col_l);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint32_t m = uint32_t(__builtin_amdgcn_ds_bpermute(src, int(mv[2 * s + h])));
          gs[cb][h] = bf16_lo(m);
          gc[cb][h] = __builtin_fmaf(-128.0f, bf16_lo(m), bf16_hi(m));
        }
      }
      if constexpr (NRB == 1) {
        // one row block: word j's (128 + q) pairs feed both groups' MFMAs
        f32x4_t pg[4][2];
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
          for (int h = 0; h < 2; ++h) pg[cb][h] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          u32x4_t b[4];
#pragma unroll
          for (int cb = 0; cb < 4; ++cb) {
            const uint32_t v = wr[cb][s][j];
#pragma unroll
            for (int r = 0; r < 4; ++r) b[cb][r] = and_or(v >> (4 * r), 0x000F000Fu, kMagic128x2);
          }
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const u32x4_t a = *reinterpret_cast<const u32x4_t*>(&xs[(gh == h ? own[j] : zoff) + 128 * s]);
#pragma unroll
            for (int cb = 0; cb < 4; ++cb)
              pg[cb][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  __builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b[cb]), pg[cb][h], 0, 0, 0);
          }
        }
        // the lane's rows 4g + r: acc += s·P + (b − 128·s)·Σx, group 2s then 2s + 1
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float2 xg = *reinterpret_cast<const float2*>(&xsum[(4 * g + r) * 8 + 2 * s]);
#pragma unroll
          for (int cb = 0; cb < 4; ++cb) {
            float v = acc[0][cb][r];
            v = __builtin_fmaf(gs[cb][0], pg[cb][0][r], v);
            v = __builtin_fmaf(gc[cb][0], xg.x, v);
            v = __builtin_fmaf(gs[cb][1], pg[cb][1][r], v);
            v = __builtin_fmaf(gc[cb][1], xg.y, v);
            acc[0][cb][r] = v;
          }
        }
      } else {
        // several row blocks: every word's (128 + q) pairs once per step, then
        // one group of one row block at a time
        u32x4_t b[4][4];   // (128 + q) pairs of word j, column block cb
  #pragma unroll
        for (int j = 0; j < 4; ++j)
  #pragma unroll
          for (int cb = 0; cb < 4; ++cb) {
            const uint32_t v = wr[cb][s][j];
  #pragma unroll
            for (int r = 0; r < 4; ++r) b[j][cb][r] = and_or(v >> (4 * r), 0x000F000Fu, kMagic128x2);
          }
  #pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
  #pragma unroll
          for (int h = 0; h < 2; ++h) {   // group 2s + h
            f32x4_t pg[4];
  #pragma unroll
            for (int cb = 0; cb < 4; ++cb) pg[cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  #pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int off = (gh == h ? own[j] + rb * 16 * kSlabCodes : zoff) + 128 * s;
              const u32x4_t a = *reinterpret_cast<const u32x4_t*>(&xs[off]);
  #pragma unroll
              for (int cb = 0; cb < 4; ++cb)
                pg[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b[j][cb]), pg[cb], 0, 0, 0);
            }
            // the lane's rows 16rb + 4g + r: acc += s·P + (b − 128·s)·Σx
  #pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float xg = xsum[(16 * rb + 4 * g + r) * 8 + 2 * s + h];
  #pragma unroll
              for (int cb = 0; cb < 4; ++cb)
                acc[rb][cb][r] = __builtin_fmaf(gc[cb][h], xg, __builtin_fmaf(gs[cb][h], pg[cb][r], acc[rb][cb][r]));
            }
          }
        }
      }
    }
  } else {
  // 3. MXFP4 (exact in bf16): per step the exponent each lane's chunk needs
  //    (from the lane that loaded that column), then per word j the four
  //    column blocks' weights and the MFMAs of every row block
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    if (128 * s >= w) break;   // a narrow last slab ends early (uniform)
    float sc[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      // group (128s + 32g) / 32 = 4s + g: byte g of dword s
      const int src = 4 * (16 * cb + col_l);
      sc[cb] = e8m0_scale((uint32_t(__builtin_amdgcn_ds_bpermute(src, int(mv[s]))) >> (8 * g)) & 0xFFu);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x4_t bf[4];
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) bf[cb] = mxfp4_word_to_bf16x8(wr[cb][s][j], sc[cb]);
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        const u32x4_t a = *reinterpret_cast<const u32x4_t*>(&xs[xs_at(16 * rb + col_l, 16 * s + 4 * g + j)]);
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
          acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, bf[cb]), acc[rb][cb], 0, 0, 0);
      }
    }
  }

  }

  // 4. this slab's partial sums: lane holds column col_l, rows 4g + r of each block
  float* plane = ws + int64_t(sl) * t * n;
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const int col = wcol + 16 * cb + col_l;
      if (col >= n) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * rb + 4 * g + r;
        if (row < t) plane[int64_t(row) * n + col] = acc[rb][cb][r];
      }
    }
  }
}

// y = bf16(Σ_slab partial), the planes added in slab order, up to eight
// planes' loads in flight per element
__global__ __launch_bounds__(256) void skinny_reduce_kernel(const float* __restrict__ ws, int64_t tn,
                                                            int slabs, uint16_t* __restrict__ y) {
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < tn; i += int64_t(gridDim.x) * 256) {
    float s = ws[i];
    for (int k0 = 1; k0 < slabs; k0 += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = k0 + u < slabs ? ws[int64_t(k0 + u) * tn + i] : 0.f;
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (k0 + u < slabs) s += v[u];
    }
    y[i] = f32_to_bf16(s);
  }
}

}  // namespace

int launch_skinny(const GemmArgs& a, float* ws, void* stream) {
  Layout l;
  if (!layout_of(a.f, a.n, a.d, &l)) return int(hipErrorInvalidValue);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint8_t* codes = a.packed + l.codes_offset;
  const uint8_t* meta = a.packed + l.meta_offset;
  const int slabs = (a.d + kSlabCodes - 1) / kSlabCodes;
  const dim3 grid(unsigned((a.n + 255) / 256), unsigned(slabs));
  const int rb = (a.t + 15) / 16;   // row blocks: 1, 2 or 4 (the launched kernel's NRB)
  const size_t lds = size_t(rb == 3 ? 4 : rb) * 16 * kSlabCodes * 2 + kSkExtraBytes;
  const uint32_t cb = uint32_t(int64_t(a.n) * (a.d / 2)), mb = uint32_t(l.meta_bytes);
  const int64_t tn = int64_t(a.t) * a.n;
  // armed profiling events: start with the first kernel, stop with the second
  const ProfileEvents pe = take_profile_events();
  const int nrb = (a.t + 15) / 16;
  auto pick = [&](auto fmt) {
    constexpr int F = decltype(fmt)::value;
    return nrb == 1 ? skinny_kernel<F, 1> : nrb == 2 ? skinny_kernel<F, 2> : skinny_kernel<F, 4>;
  };
  auto k1 = a.f == QMM_AFFINE4_G64 ? pick(std::integral_constant<int, QMM_AFFINE4_G64>{})
                                   : pick(std::integral_constant<int, QMM_MXFP4_G32>{});
  if (pe.start)
    hipExtLaunchKernelGGL(k1, grid, dim3(256), uint32_t(lds), s, static_cast<hipEvent_t>(pe.start), nullptr, 0,
                          codes, meta, cb, mb, a.t, a.n, a.d, a.x, ws);
  else
    hipLaunchKernelGGL(k1, grid, dim3(256), lds, s, codes, meta, cb, mb, a.t, a.n, a.d, a.x, ws);
  launch_partials_sum(ws, tn, slabs, a.y, pe.stop, s);
  return int(hipGetLastError());
}

void launch_partials_sum(const float* ws, int64_t tn, int planes, uint16_t* y, void* stop, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const unsigned grid = unsigned(std::min<int64_t>((tn + 255) / 256, 4096));
  if (stop)
    hipExtLaunchKernelGGL(skinny_reduce_kernel, dim3(grid), dim3(256), 0, s, nullptr, static_cast<hipEvent_t>(stop),
                          0, ws, tn, planes, y);
  else
    hipLaunchKernelGGL(skinny_reduce_kernel, dim3(grid), dim3(256), 0, s, ws, tn, planes, y);
}

}  // namespace qmm
