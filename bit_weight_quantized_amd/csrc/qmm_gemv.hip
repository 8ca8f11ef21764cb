// Decode GEMV y = Ŵ·x for 4-bit weights on gfx950, dense and grouped (one
// launch over all routed experts).
//
// Work split.  A wave owns one quad of 4 consecutive output rows across the
// whole reduction axis; lane l works on row (l / 16) of the quad and on the
// 32-code chunk (l % 16) of the current 512-code slab.  With the K-slabbed
// packed layout the quad's 4 rows of one slab are 1 KiB contiguous, so each
// wave code load is one contiguous 1 KiB, and since every wave walks the slabs
// in the same order the whole GPU sweeps the weights front to back like a
// streaming copy.  A matrix with few quads (n <= 6144) would leave most of
// the chip with one short chain of slab loads per wave, so there the quad's
// slabs are dealt to WQ = 2 or 4 waves of the workgroup (slab s to wave
// s % WQ), each lane's per-slab partial sum goes to LDS, and one wave adds them
// in slab order exactly as a single wave adds them in registers: the result is
// bit for bit the same whatever WQ.
//
// Load order.  A wave's vector-memory loads complete in issue order, and a
// wait names how many may still be outstanding, so every load is issued
// unconditionally (a load that must not happen gets an out-of-range buffer
// offset and returns zeros) and in the order it is consumed: first the
// activation pieces and the quad's metadata for the pass, then a ring of kRing
// code slabs.  Consuming slab s waits only for slab s; its ring slot is then
// refilled with slab s + kRing.
//
// Activations and metadata are staged in LDS once per pass of up to
// kPassSlabs slabs: the workgroup's activation row, cut into 32-code chunks
// of 80 bytes (64 bytes of bf16, the chunk's sum at +64), and each wave's
// metadata for its quad (one contiguous piece of the quad-major metadata,
// copied as it lies: slab by slab, row by row).
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

#include "qmm_device.h"
#include "qmm_internal.h"
#include "qmm_launch.h"

namespace qmm {
namespace {

constexpr int kWaves = 4;                 // waves per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kRing = 3;                  // code slabs in flight per lane (3 KiB per wave)
constexpr int kPassSlabs = 12;            // slabs staged in LDS per pass
constexpr int kChunkBytes = 80;           // LDS activation chunk: 64 B of x, sum at +64
constexpr int kXL = kPassSlabs * 64 / kThreads;   // 16-byte activation pieces per thread
static_assert(kPassSlabs * 64 % kThreads == 0, "activation pieces must divide evenly");

// metadata bytes of one quad (4 rows) in a full slab, loaded as 16-byte pieces
template <int FMT>
constexpr int quad_meta_bytes() { return FMT == QMM_AFFINE4_G64 ? 128 : 64; }
template <int FMT>
constexpr int meta_pieces_per_lane() { return (kPassSlabs * quad_meta_bytes<FMT>() / 16 + 63) / 64; }

constexpr uint32_t kOOB = 0x80000000u;    // OR-ed into a buffer offset: past every range

__device__ __forceinline__ u32x4_t ld16_stream(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  // weights are read once: non-temporal, so they do not displace reused lines
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, int(off), 0, 2));
}
__device__ __forceinline__ u32x4_t ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, int(off), 0, 0));
}

template <int FMT>
__device__ __forceinline__ float chunk_partial(const u32x4_t w, const uint8_t* xc, uint32_t m) {
  const u32x4_t v0 = *reinterpret_cast<const u32x4_t*>(xc);
  const u32x4_t v1 = *reinterpret_cast<const u32x4_t*>(xc + 16);
  const u32x4_t v2 = *reinterpret_cast<const u32x4_t*>(xc + 32);
  const u32x4_t v3 = *reinterpret_cast<const u32x4_t*>(xc + 48);
  uint32_t xp[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    xp[i] = v0[i];
    xp[4 + i] = v1[i];
    xp[8 + i] = v2[i];
    xp[12 + i] = v3[i];
  }
  if (FMT == QMM_AFFINE4_G64) {
    const float xsum = *reinterpret_cast<const float*>(xc + 64);
    const float dot = affine_dot32(w, xp);
    const float sc = bf16_lo(m), bi = bf16_hi(m);
    return __builtin_fmaf(sc, __builtin_fmaf(-128.f, xsum, dot), bi * xsum);
  }
  return __builtin_ldexpf(mxfp4_dot32(w, xp), int(m) - 127);
}

template <int FMT, bool GROUPED, int WQ>
__global__ __launch_bounds__(kThreads) void gemv_kernel(
    const uint8_t* __restrict__ base, int64_t expert_stride, int n_experts, int64_t codes_off,
    int64_t meta_off, uint32_t codes_bytes, uint32_t meta_bytes, int n, int d,
    const uint16_t* __restrict__ x, int64_t t_x, const int32_t* __restrict__ row_index,
    const int32_t* __restrict__ seg_expert, const int32_t* __restrict__ seg_offsets, int m_total,
    uint16_t* __restrict__ y) {
  constexpr int QMB = quad_meta_bytes<FMT>();
  constexpr int ML = meta_pieces_per_lane<FMT>();
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const Slabs L{n, d, FMT};
  const int nslabs = L.count();
  // LDS: activation chunks of one pass, a trash slot, each wave's metadata, a trash slot
  const int pslabs = min(nslabs, kPassSlabs);
  const uint32_t x_trash = uint32_t(pslabs) * 16u * kChunkBytes;
  const uint32_t m_base = x_trash + 16u;
  const uint32_t m_wave = uint32_t(pslabs) * QMB;
  const uint32_t m_trash = m_base + kWaves * m_wave;
  // WQ > 1: per-slab partial sums of the pass, [slab][quad of the workgroup][lane],
  // after the metadata trash slot
  constexpr int QPW = kWaves / WQ;   // quads per workgroup
  float* red = reinterpret_cast<float*>(smem + m_trash + 16u);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rsub = lane >> 4, c = lane & 15;
  const int wk = wave % WQ;           // this wave's share of the quad's slabs: s % WQ == wk
  const int ql = wave / WQ;
  const int quad = blockIdx.x * QPW + ql;
  const int row = quad * 4 + rsub;
  const int lrow = min(row, n - 1);   // rows past n (last quad only) load row n - 1, store nothing

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
  const __amdgpu_buffer_rsrc_t cr = make_rsrc(blob + codes_off, codes_bytes);
  const __amdgpu_buffer_rsrc_t mr = make_rsrc(blob + meta_off, meta_bytes);
  const uint8_t* mwave = smem + m_base + wave * m_wave;

  for (int gr = r_begin; gr < r_end; ++gr) {
    const uint16_t* xrow = x;
    uint16_t* yrow = y;
    bool bad_row = false;
    if (GROUPED) {
      const int src = row_index[gr];
      bad_row = bad_expert || src < 0 || src >= t_x;
      xrow = x + (bad_row ? 0 : int64_t(src) * d);
      yrow = y + int64_t(gr) * n;
    }
    float acc = 0.f;
    for (int p0 = 0; p0 < nslabs; p0 += kPassSlabs) {
      const int ps = min(kPassSlabs, nslabs - p0);   // slabs in this pass
      const int k0 = p0 * kSlabCodes;
      // 1. activation pieces of the pass (zeros past d)
      const __amdgpu_buffer_rsrc_t xr = make_rsrc(xrow + k0, uint32_t(d - k0) * 2u);
      u32x4_t xv[kXL];
#pragma unroll
      for (int i = 0; i < kXL; ++i) xv[i] = ld16(xr, 16u * uint32_t(tid + i * kThreads));
      // 2. the quad's metadata for the pass: one contiguous piece (quad-major layout)
      const uint32_t m0 = uint32_t(quad) * uint32_t(L.meta_quad()) + uint32_t(p0 * QMB);
      const int mbytes = (ps - 1) * QMB + 4 * L.meta_row(p0 + ps - 1);
      u32x4_t mv[ML];
#pragma unroll
      for (int i = 0; i < ML; ++i) {
        const int pc = lane + 64 * i;
        const bool mine = WQ == 1 || (16 * pc / QMB) % WQ == wk;
        mv[i] = ld16(mr, 16 * pc < mbytes && mine ? m0 + 16u * pc : kOOB);
      }
      // 3. the code ring: this lane's chunk of slab s (zeros past the slab's width)
      // the wave's i-th slab of the pass is slab wk + WQ·i
      const int cnt = ps > wk ? (ps - wk + WQ - 1) / WQ : 0;
      auto code_off = [&](int i) -> uint32_t {
        const int sg = p0 + wk + WQ * i;
        if (i >= cnt) return kOOB;
        return 32 * c < L.width(sg) ? uint32_t(L.codes(sg, lrow)) + 16u * c : kOOB;
      };
      u32x4_t ring[kRing];
#pragma unroll
      for (int j = 0; j < kRing; ++j) ring[j] = ld16_stream(cr, code_off(j));
      // 4. stage activations and metadata (pieces past the pass go to the trash slots)
#pragma unroll
      for (int i = 0; i < kXL; ++i) {
        const int pc = tid + i * kThreads;
        const uint32_t dst = pc < ps * 64 ? uint32_t(pc >> 2) * kChunkBytes + 16u * (pc & 3) : x_trash;
        *reinterpret_cast<u32x4_t*>(smem + dst) = xv[i];
      }
#pragma unroll
      for (int i = 0; i < ML; ++i) {
        const int pc = lane + 64 * i;
        const uint32_t dst = 16 * pc < mbytes ? m_base + wave * m_wave + 16u * pc : m_trash;
        *reinterpret_cast<u32x4_t*>(smem + dst) = mv[i];
      }
      __syncthreads();
      if (FMT == QMM_AFFINE4_G64) {
        if (tid < ps * 16) {
          const uint8_t* p = smem + tid * kChunkBytes;
          float a = 0.f, b = 0.f;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const u32x4_t v = *reinterpret_cast<const u32x4_t*>(p + 16 * j);
            a = dot2_bf16(v[0], 0x3F803F80u, a);   // (1.0, 1.0)
            b = dot2_bf16(v[1], 0x3F803F80u, b);
            a = dot2_bf16(v[2], 0x3F803F80u, a);
            b = dot2_bf16(v[3], 0x3F803F80u, b);
          }
          *reinterpret_cast<float*>(smem + tid * kChunkBytes + 64) = a + b;
        }
        __syncthreads();
      }
      // 5. consume the wave's i-th slab from ring slot i % kRing, refill the slot
      //    with its slab i + kRing
      for (int i0 = 0; i0 < cnt; i0 += kRing) {
#pragma unroll
        for (int j = 0; j < kRing; ++j) {
          const int i = i0 + j;
          if (i < cnt) {
            const int s = wk + WQ * i;
            const int sg = p0 + s;
            const uint8_t* mp = mwave + s * QMB + rsub * L.meta_row(sg);
            const uint32_t m = FMT == QMM_AFFINE4_G64
                                   ? *reinterpret_cast<const uint32_t*>(mp + 4 * (c >> 1))
                                   : uint32_t(mp[c]);
            const float part = chunk_partial<FMT>(ring[j], smem + (s * 16 + c) * kChunkBytes, m);
            // chunks past a narrow last slab hold no weights (their metadata is not staged)
            const float pv = 32 * c < L.width(sg) ? part : 0.f;
            if constexpr (WQ == 1)
              acc += pv;
            else
              red[(s * QPW + ql) * 64 + lane] = pv;
          }
          ring[j] = ld16_stream(cr, code_off(i + kRing));
        }
      }
      if constexpr (WQ > 1) {
        // the pass's slab partials added in slab order, as one wave would
        __syncthreads();
        if (wk == 0)
          for (int s = 0; s < ps; ++s) acc += red[(s * QPW + ql) * 64 + lane];
      }
      if (p0 + kPassSlabs < nslabs || (GROUPED && gr + 1 < r_end)) __syncthreads();
    }
    const float v = sum16(acc);
    if (wk == 0 && c == 0 && row < n) yrow[row] = f32_to_bf16((GROUPED && bad_row) ? __builtin_nanf("") : v);
  }
}

template <int FMT, bool GROUPED, int WQ>
void launch_fmt(const GemvArgs& a, const Layout& l, dim3 grid, hipStream_t s) {
  const uint32_t codes_bytes = uint32_t(int64_t(a.n) * (a.d / 2));
  const uint32_t meta_bytes = uint32_t(l.meta_bytes);
  const int nslabs = (a.d + kSlabCodes - 1) / kSlabCodes;
  const int ps = nslabs < kPassSlabs ? nslabs : kPassSlabs;
  const size_t lds = size_t(ps) * 16 * kChunkBytes + 16 + size_t(kWaves) * ps * quad_meta_bytes<FMT>() + 16 +
                     (WQ > 1 ? size_t(ps) * (kWaves / WQ) * 64 * 4 : 0);
  launch_kernel_lds((gemv_kernel<FMT, GROUPED, WQ>), grid, dim3(kThreads), lds, s, a.packed,
                    a.expert_stride, a.n_experts, l.codes_offset, l.meta_offset, codes_bytes,
                    meta_bytes, a.n, a.d, a.x, a.t_x, a.row_index, a.seg_expert, a.seg_offsets,
                    a.m_total, a.y);
}

}  // namespace

int launch_gemv(const GemvArgs& a, void* stream) {
  Layout l;
  if (!layout_of(a.f, a.n, a.d, &l)) return int(hipErrorInvalidValue);
  // 32-bit buffer offsets: one blob's codes and metadata must stay under 2 GiB
  if (int64_t(a.n) * (a.d / 2) >= (int64_t(1) << 31) || l.meta_bytes >= (int64_t(1) << 31))
    return int(hipErrorInvalidValue);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int nseg = a.n_seg > 0 ? a.n_seg : 1;
  // waves per quad: a few quads (measured at d = 5120: n = 512 .. 5120 gain
  // 0.4 - 0.6 µs of 4 - 6 µs with four waves per quad; 7168 and 13824 lose
  // with any split) are split along K while each wave keeps two slabs or more
  const int quads = (a.n + 3) / 4;
  const int nslabs = (a.d + kSlabCodes - 1) / kSlabCodes;
  const int wq = a.n_seg > 0 || quads > 1536 ? 1 : nslabs >= 8 ? 4 : nslabs >= 4 ? 2 : 1;
  dim3 grid(unsigned((int64_t(quads) * wq + kWaves - 1) / kWaves), unsigned(nseg));
  if (a.n_seg > 0) {
    if (a.f == QMM_AFFINE4_G64)
      launch_fmt<QMM_AFFINE4_G64, true, 1>(a, l, grid, s);
    else
      launch_fmt<QMM_MXFP4_G32, true, 1>(a, l, grid, s);
  } else if (wq == 4) {
    if (a.f == QMM_AFFINE4_G64)
      launch_fmt<QMM_AFFINE4_G64, false, 4>(a, l, grid, s);
    else
      launch_fmt<QMM_MXFP4_G32, false, 4>(a, l, grid, s);
  } else if (wq == 2) {
    if (a.f == QMM_AFFINE4_G64)
      launch_fmt<QMM_AFFINE4_G64, false, 2>(a, l, grid, s);
    else
      launch_fmt<QMM_MXFP4_G32, false, 2>(a, l, grid, s);
  } else {
    if (a.f == QMM_AFFINE4_G64)
      launch_fmt<QMM_AFFINE4_G64, false, 1>(a, l, grid, s);
    else
      launch_fmt<QMM_MXFP4_G32, false, 1>(a, l, grid, s);
  }
  return int(hipGetLastError());
}

}  // namespace qmm
