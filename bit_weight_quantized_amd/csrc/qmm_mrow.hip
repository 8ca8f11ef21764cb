// Multi-row GEMV: Y = X·Ŵᵀ for 2 <= T <= 64 activation rows (a batch of
// decode tokens), the product of "Kapitsa 源码拆解 02：权重、矩阵与 Metal",
// section "矩阵乘法中数据和参数", at a size where every weight byte is read once
// and serves all T rows, with no partial sums in memory and no second kernel.
//
// Work split.  The columns are dealt out evenly to a multiple of the CU count
// of workgroups (one resident per CU), at most 128 columns each.  A wave owns
// 16 columns; the workgroup's column waves are repeated kq times (8 waves in
// all), wave group kq taking slabs kq, kq + KQ, ... of d with two slabs in
// flight per lane, and the groups' partial sums meet in LDS in a fixed order.
// Each workgroup first copies the T activation rows (zeros past d, padded to
// whole slabs) to LDS by DMA, 16-byte pieces swizzled within each 256-byte
// group so that the 16 rows of one MFMA operand read sit in distinct banks
// (more than 16 rows do not fit: they take the streaming form further down).
// The rows enter v_mfma_f32_16x16x32_bf16 as its 16-row A operand (rows past
// T read row T - 1 and their outputs are dropped); lane (column c, chunk g)
// loads the 32-code chunk g of each 128-code step of its column.
//
// Affine weights enter as the exact bf16 values 128 + q and each 64-code
// group's scale and bias follow in fp32: s·Σx(128 + q) + (b − 128·s)·Σx, with
// Σx per row and group summed once per workgroup.  A step's two groups are
// kept apart by regrouping the loaded words across lanes (v_permlane32_swap)
// so that every MFMA sees one group.  MXFP4 weights convert exactly to bf16
// with their E8M0 scale.  No weight is rounded.
//
// Grouped form (routed experts, a few rows per segment): the same kernel with
// blockIdx.y a segment of the routing tables, its expert's weights, and its
// rows gathered through row_index; a segment longer than the launch's T rows
// takes several passes, each re-reading the expert.
#include <hip/hip_runtime.h>

#include "qmm_device.h"
#include "qmm_internal.h"
#include "qmm_launch.h"
#include "qmm_lds_copy.h"
#include "qmm_mrow.h"

namespace qmm {
namespace {

constexpr uint32_t kOOB = 0x80000000u;   // OR-ed into a buffer offset: past every range
constexpr int kMrRing = 2;               // slabs in flight per lane

// element offset of 16-byte piece c of row r (row stride rs elements)
__device__ __forceinline__ int mr_at(int r, int rs, int c) { return r * rs + ((c ^ (r & 15)) << 3); }

template <int FMT, int KQ, bool G2, bool GRP, bool GLU = false>
__global__ __launch_bounds__(64 * kMrowMaxWaves) void mrow_kernel(const uint8_t* __restrict__ codes,
                                                   const uint8_t* __restrict__ meta,
                                                   uint32_t codes_bytes, uint32_t meta_bytes, int t,
                                                   int n, int d, int cpw, int ncw,
                                                   const uint16_t* __restrict__ x,
                                                   uint16_t* __restrict__ y, MrowGroups grp) {
  constexpr bool AFF = FMT == QMM_AFFINE4_G64;
  static_assert(!G2 || AFF, "two groups per MFMA: affine weights only");
  static_assert(!GLU || (GRP && KQ == 1), "the activation: grouped, one wave per column block");
  constexpr int MP = AFF ? 2 : 1;   // 16-byte metadata pieces of one column per slab
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];
  const Slabs L{n, d, FMT};
  const int ns = L.count();
  const int rs = ns * kSlabCodes;   // LDS row stride in elements (rows padded to whole slabs)
  const int ng = ns * 8;            // 64-code groups per padded row
  const int xrows = t + (G2 ? 1 : 0);   // G2: a row of zeros after the t rows
  float* xsum = reinterpret_cast<float*>(xs + xrows * rs);   // [ng][16 rows] (affine; rows past t zero)
  f32x4_t* red = reinterpret_cast<f32x4_t*>(xsum + (AFF ? ng * 16 : 0));   // [KQ - 1][ncw][64]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nw = ncw * KQ;                    // waves in the workgroup
  const int cw = wave % ncw, kq = wave / ncw;   // column block of the wave, its share of the slabs
  const int col_l = lane & 15, g = lane >> 4;
  // the workgroup's columns [c0, c1), at most 16·ncw: wave cw takes c0 + 16cw ..
  // c0 + 16cw + 15; a lane past c1 re-reads column c1 - 1 and stores nothing,
  // a wave wholly past it loads nothing.  GLU (a gate_up stack: rows [0, n/2)
  // the gate, [n/2, n) the up projection; eight waves): output columns
  // [c0, c1) of n/2, at most 64, waves 0-3 on their gate rows and waves 4-7 on
  // the same columns' up rows
  const int nout = GLU ? n / 2 : n;
  const int cwo = GLU ? cw & 3 : cw;   // the wave's column block among the outputs
  const int c0 = blockIdx.x * cpw, c1 = min(c0 + cpw, nout);
  const int col = c0 + 16 * cwo + col_l;
  const int lcol = (GLU ? (cw >> 2) * nout : 0) + min(col, c1 - 1);   // packed row the lane reads
  const bool active = 16 * cwo < c1 - c0;
  // grouped (routed experts): the workgroup's segment blockIdx.y, its rows
  // [r_begin, r_end) taken t at a time, its expert's weights; a segment with
  // no rows, or more than grp.max_rows when that is set, returns before any
  // barrier, the whole workgroup alike
  int r_begin = 0, r_end = t;
  bool bad_expert = false;
  if constexpr (GRP) {
    const int sg = blockIdx.y;
    r_begin = min(max(grp.seg_offsets[sg], 0), grp.m_total);
    r_end = min(max(grp.seg_offsets[sg + 1], r_begin), grp.m_total);
    if (r_begin >= r_end || (grp.max_rows > 0 && r_end - r_begin > grp.max_rows)) return;
    const int e = grp.seg_expert[sg];
    bad_expert = e < 0 || e >= grp.n_experts;
    const int64_t eo = bad_expert ? 0 : int64_t(e) * grp.expert_stride;
    codes += eo;
    meta += eo;
  }
  // grouped: the x row of each row of the chunk (< 0: none, or a NaN output
  // row), after the partial sums
  int* src_rows = reinterpret_cast<int*>(reinterpret_cast<char*>(red) + kMrowRedBytes);
  const __amdgpu_buffer_rsrc_t crs = make_rsrc(codes, codes_bytes);
  const __amdgpu_buffer_rsrc_t mrs = make_rsrc(meta, meta_bytes);
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(x, uint32_t(GRP ? grp.t_x : t) * uint32_t(d) * 2u);
  uint32_t pmask, pmagic;   // see step 4
  asm volatile("s_mov_b32 %0, 0x000f000f" : "=s"(pmask));
  asm volatile("v_mov_b32 %0, 0x43004300" : "=v"(pmagic));

  // the rows in chunks of at most t (one chunk when not grouped)
  for (int mb = r_begin; mb < r_end; mb += t) {
    const int tr = min(t, r_end - mb);   // rows of this chunk
    if constexpr (GRP) {
      if (tid < t) {
        int src = -1;
        if (tid < tr) {
          src = grp.row_index ? grp.row_index[mb + tid] : mb + tid;
          if (bad_expert || src < 0 || src >= grp.t_x) src = -2;
        }
        src_rows[tid] = src;
      }
      __syncthreads();
    }

    // 1. the activation rows to LDS by DMA, no registers involved: copy i of
    //    the workgroup fills LDS bytes [1024i, 1024i + 1024), lane l slot
    //    q = 64i + l, that is row r = q / (rs/8), position c' = q % (rs/8), which
    //    holds piece c = c' ^ (r & 15) of the row (zeros past d, and in the
    //    zero row)
    const int prow = rs / 8;   // 16-byte pieces per row, a multiple of 64
    const uint32_t xbase = lds_addr(xs);
    for (int i = wave; i < xrows * prow / 64; i += nw) {
      const int q = 64 * i + lane, r = q / prow, c = (q - r * prow) ^ (r & 15);
      const int sr = GRP ? (r < tr ? src_rows[r] : -1) : r;   // the x row (grouped: gathered)
      copy16_to_lds(xrs, r < tr && sr >= 0 && 8 * c < d ? (uint32_t(sr) * uint32_t(d) + 8u * uint32_t(c)) * 2u : kOOB,
                    xbase + 1024u * uint32_t(i));
    }

    // 2. the code ring over the wave's slabs kq, kq + KQ, kq + 2KQ, ...: slab
    //    s's four pieces (step j: codes 128j + 32g .. +31 of the slab) and its
    //    metadata, issued in the order they are used
    u32x4_t rc[kMrRing][4];
    u32x4_t rm[kMrRing][MP];
    auto issue = [&](u32x4_t (&c4)[4], u32x4_t (&m)[MP], int s) {
      const bool in = active && s < ns;
      const int w = in ? L.width(s) : 0;
      const uint32_t cb = in ? uint32_t(L.codes(s, lcol)) : 0u;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kk = 128 * j + 32 * g;
        c4[j] = buf_load16(crs, kk < w ? cb + uint32_t(kk >> 1) : kOOB);
      }
      const int mrow = in ? L.meta_row(s) : 0;
      const uint32_t mb = in ? uint32_t(L.meta(s, lcol)) : 0u;
#pragma unroll
      for (int i = 0; i < MP; ++i) m[i] = buf_load16(mrs, 16 * i < mrow ? mb + 16u * uint32_t(i) : kOOB);
    };
#pragma unroll
    for (int j = 0; j < kMrRing; ++j) issue(rc[j], rm[j], kq + j * KQ);

    // 3. the wave's copies landed: they were issued before the ring, so the
    //    wait the compiler places for the first slab (its own loads, which it
    //    counts) covers them; then every wave's copies are visible
    asm volatile("" ::"v"(rc[0][0]), "v"(rc[0][1]), "v"(rc[0][2]), "v"(rc[0][3]), "v"(rm[0][0]), "v"(rm[0][MP - 1]));
    __syncthreads();
    if constexpr (AFF) {
      // each row's sum over each 64-code group (consecutive threads take
      // consecutive rows of one group: their pieces sit in distinct banks)
      for (int q = tid; q < ng * 16; q += 64 * nw) {
        const int r = q & 15, gr = q >> 4;
        float sum[4] = {0.f, 0.f, 0.f, 0.f};   // four chains: dword k of every piece
        if (r < tr) {
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            const u32x4_t v = *reinterpret_cast<const u32x4_t*>(&xs[mr_at(r, rs, 8 * gr + c)]);
            // each pair of the dword as a bf16 dot against (1, 1)
#pragma unroll
            for (int k = 0; k < 4; ++k) sum[k] = dot2_bf16(v[k], 0x3F803F80u, sum[k]);
          }
        }
        xsum[q] = (sum[0] + sum[1]) + (sum[2] + sum[3]);
      }
      __syncthreads();
    }

    // 4. the slabs: MFMA A operands from LDS (row col_l, clamped to the last
    //    row), B operands from the ring
    // (128 + q) pairs as (w & mask) | magic: one v_and_or_b32 that the compiler
    // emits itself once the two constants sit in registers it cannot fold back
    // into literals (an inline-asm v_and_or_b32 would get no wait states before
    // the MFMA that reads its result)
    // the lane's A-operand pieces: piece 16k + p0 (p0 < 16) of row r sits at
    // 16k + (p0 ^ (r & 15)), so each address is a per-lane base plus the
    // step's uniform offset.  MXFP4 and G2: p0 = 4g + j, word j of the lane's
    // chunk; affine otherwise: p0 = 8h + 4(g & 1) + 2 + jj − 2(g >> 1) (see the
    // regrouping below).  G2 (t <= 8): the MFMA's rows 0..7 are the x rows
    // against group 2st of the step, rows 8..15 the same x rows against group
    // 2st + 1; A row i reads x row i & 7 on the lanes of its group's chunks
    // (g >> 1 == i >> 3) and the zero row on the others.
    const int arow = G2 ? ((col_l >> 3) == (g >> 1) ? min(col_l & 7, tr - 1) : tr) : min(col_l, tr - 1);
    int aoff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p0 = AFF && !G2 ? 8 * (i >> 1) + 4 * (g & 1) + 2 + (i & 1) - 2 * (g >> 1) : 4 * g + i;
      aoff[i] = arow * rs + ((p0 ^ (arow & 15)) << 3);
    }
    f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
    auto slab = [&](const u32x4_t (&c4)[4], const u32x4_t (&m)[MP], int s) {
      const int w = L.width(s);
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        if (128 * st >= w) break;   // a narrow last slab ends early (uniform)
        const int e0 = (s * 64 + st * 16) * 8;   // the step's first activation element
        if constexpr (G2) {
          // the lane's chunk g lies in group 2st + h, h = g >> 1; its rows
          // 4(g & 1) .. + 3 of the MFMA sum that group only (the narrow last
          // slab's missing second group: zero metadata, zero sums)
          const int h = g >> 1;
          const uint32_t mh = h ? (128 * st + 64 < w ? m[st >> 1][(2 * st + 1) & 3] : 0u) : m[st >> 1][(2 * st) & 3];
          const float gs = bf16_lo(mh), gc = __builtin_fmaf(-128.0f, bf16_lo(mh), bf16_hi(mh));
          f32x4_t pg = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            u32x4_t b;
#pragma unroll
            for (int r = 0; r < 4; ++r) b[r] = ((c4[st][j] >> (4 * r)) & pmask) | pmagic;
            const u32x4_t a = *reinterpret_cast<const u32x4_t*>(&xs[aoff[j] + e0]);
            pg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                         __builtin_bit_cast(bf16x8_t, b), pg, 0, 0, 0);
          }
          // acc += s·P + (b − 128·s)·Σx for x rows 4(g & 1) + r, group 2st + h
          const f32x4_t xg = *reinterpret_cast<const f32x4_t*>(&xsum[(s * 8 + 2 * st + h) * 16 + 4 * (g & 1)]);
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[r] = __builtin_fmaf(gc, xg[r], __builtin_fmaf(gs, pg[r], acc[r]));
        } else if constexpr (AFF) {
          // groups 2st and 2st + 1 of the slab: dwords 2st, 2st + 1 of the column's metadata
          // (a last slab may end after group 2st: its second group's dword
          // belongs to another column and is replaced by zero)
          const uint32_t m0 = m[st >> 1][(2 * st) & 3];
          const uint32_t m1 = 128 * st + 64 < w ? m[st >> 1][(2 * st + 1) & 3] : 0u;
          const float gs0 = bf16_lo(m0), gc0 = __builtin_fmaf(-128.0f, bf16_lo(m0), bf16_hi(m0));
          const float gs1 = bf16_lo(m1), gc1 = __builtin_fmaf(-128.0f, bf16_lo(m1), bf16_hi(m1));
          // regroup the step's words so that each register holds one group in
          // every lane: lanes 32..63 (chunks 2, 3: group 2st + 1) trade word J - 2
          // for word J (J = 2, 3) of lanes 0..31 (chunks 0, 1: group 2st), the
          // same column.  Then wg[0][*] is group 2st, wg[1][*] group 2st + 1, and
          // lane g's word wg[h][J - 2] holds the codes of piece
          // 8h + 4(g & 1) + J - 2(g >> 1) of the step.
          const auto s20 = __builtin_amdgcn_permlane32_swap(c4[st][2], c4[st][0], false, false);
          const auto s31 = __builtin_amdgcn_permlane32_swap(c4[st][3], c4[st][1], false, false);
          const uint32_t wg[2][2] = {{s20[0], s31[0]}, {s20[1], s31[1]}};
          f32x4_t pg[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
              u32x4_t b;
#pragma unroll
              for (int r = 0; r < 4; ++r) b[r] = ((wg[h][jj] >> (4 * r)) & pmask) | pmagic;
              const u32x4_t a = *reinterpret_cast<const u32x4_t*>(&xs[aoff[2 * h + jj] + e0]);
              pg[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                              __builtin_bit_cast(bf16x8_t, b), pg[h], 0, 0, 0);
            }
          // the lane's rows 4g + r: acc += s·P + (b − 128·s)·Σx, group 2st then 2st + 1
          const f32x4_t xg0 = *reinterpret_cast<const f32x4_t*>(&xsum[(s * 8 + 2 * st) * 16 + 4 * g]);
          const f32x4_t xg1 = *reinterpret_cast<const f32x4_t*>(&xsum[(s * 8 + 2 * st + 1) * 16 + 4 * g]);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float v = acc[r];
            v = __builtin_fmaf(gs0, pg[0][r], v);
            v = __builtin_fmaf(gc0, xg0[r], v);
            v = __builtin_fmaf(gs1, pg[1][r], v);
            v = __builtin_fmaf(gc1, xg1[r], v);
            acc[r] = v;
          }
        } else {
          // group 4st + g of the slab: byte 4st + g of the column's metadata
          const float sc = e8m0_scale((m[0][st] >> (8 * g)) & 0xFFu);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const u32x4_t a = *reinterpret_cast<const u32x4_t*>(&xs[aoff[j] + e0]);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                          __builtin_bit_cast(bf16x8_t, mxfp4_word_to_bf16x8(c4[st][j], sc)),
                                                          acc, 0, 0, 0);
          }
        }
      }
    };
    for (int s0 = kq; active && s0 < ns; s0 += kMrRing * KQ) {
#pragma unroll
      for (int j = 0; j < kMrRing; ++j) {
        const int s = s0 + j * KQ;
        if (s < ns) slab(rc[j], rm[j], s);
        issue(rc[j], rm[j], s + kMrRing * KQ);
      }
    }

    // 5. G2: lanes g and g ^ 2 hold the two halves of x rows 4(g & 1) + r
    //    (groups 2st and 2st + 1 of every step): added, the first half first
    if constexpr (G2) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[r]), __float_as_uint(acc[r]), false, false);
        acc[r] = lane < 32 ? acc[r] + __uint_as_float(sw[1]) : __uint_as_float(sw[0]) + acc[r];
      }
    }
    // 6. the KQ shares of each column block summed in order kq = 0, 1, ...;
    //    lane holds column col, rows 4g .. 4g + 3 (G2: rows 4(g & 1) + r, g < 2)
    if constexpr (KQ > 1) {
      if (kq > 0) red[((kq - 1) * ncw + cw) * 64 + lane] = acc;
      __syncthreads();
      if (kq == 0) {
#pragma unroll
        for (int k = 1; k < KQ; ++k) acc += red[((k - 1) * ncw + cw) * 64 + lane];
      }
    }
    if constexpr (GLU) {
      // the up waves hand their sums to the gate waves of the same columns
      // (through the partial-sum area, unused with one wave per column block),
      // which store h = silu(gate)·up, rounded once
      if (cw >= 4) red[(cw - 4) * 64 + lane] = acc;
      __syncthreads();
      if (cw < 4 && col < c1 && (!G2 || g < 2)) {
        const f32x4_t u = red[cw * 64 + lane];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 4 * (G2 ? g & 1 : g) + r;
          if (row < tr) {
            const float gv = acc[r];
            const float h = gv / (1.0f + expf(-gv)) * u[r];
            y[int64_t(mb + row) * nout + col] = f32_to_bf16(src_rows[row] < 0 ? __builtin_nanf("") : h);
          }
        }
      }
    } else if (kq == 0 && col < c1 && (!G2 || g < 2)) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 4 * (G2 ? g & 1 : g) + r;
        if (row < tr) {
          const float v = GRP && src_rows[row] < 0 ? __builtin_nanf("") : acc[r];
          y[int64_t(mb + row) * n + col] = f32_to_bf16(v);
        }
      }
    }
    if constexpr (GRP) __syncthreads();   // the next chunk rewrites the rows, the sums and the partials
  }
}

// Streaming form for 17 <= T <= 64 rows (RB = ceil(T / 16) row blocks of the
// MFMA's 16-row A operand): the rows no longer fit in LDS whole, so they pass
// through two slab buffers.  Eight waves: four column waves of 16 columns (up
// to 64 columns per workgroup) times two halves of each slab (its 128-code
// steps 0, 1 and 2, 3), the two halves' sums meeting in LDS at the end.  Each
// lane keeps its half of four slabs' codes in flight, and the workgroup the
// rows of the next two slabs: while slab s is multiplied from one buffer,
// the rows of slab s + 2 are loaded into registers and those of slab s + 1,
// which landed meanwhile, are stored into the other buffer (zeros past T and
// past d), with their affine group sums taken on the way (bf16 dots against
// (1, 1), then across the eight lanes of a group); one
// barrier per slab.  Every weight is read once for all rows and each of its
// operands feeds RB MFMAs.
constexpr int kStRing = 4;   // slabs of codes in flight per lane
constexpr int kStXd = 2;     // slabs of rows in flight (divides kStRing)
static_assert(kStRing % 2 == 0 && kStRing % kStXd == 0, "buffer and ring slots repeat every kStRing slabs");

template <int FMT, int RB>
__global__ __launch_bounds__(512) void mrow_stream_kernel(const uint8_t* __restrict__ codes,
                                                          const uint8_t* __restrict__ meta,
                                                          uint32_t codes_bytes, uint32_t meta_bytes, int t,
                                                          int n, int d, int cpw,
                                                          const uint16_t* __restrict__ x,
                                                          uint16_t* __restrict__ y) {
  constexpr bool AFF = FMT == QMM_AFFINE4_G64;
  constexpr int XR = 16 * RB;             // rows of a slab buffer
  constexpr int XB = XR * kSlabCodes;     // elements of a slab buffer
  constexpr int XP = XR * 64 / 512;       // 16-byte pieces of a slab per thread
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];
  float* xsum = reinterpret_cast<float*>(xs + 2 * XB);   // affine: [buffer][group][row]
  const Slabs L{n, d, FMT};
  const int ns = L.count();

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int cw = wave & 3, kh = wave >> 2;   // column wave, half of the slab
  const int col_l = lane & 15, g = lane >> 4;
  const int c0 = blockIdx.x * cpw, c1 = min(c0 + cpw, n);
  const int col = c0 + 16 * cw + col_l;
  const int lcol = min(col, c1 - 1);
  const bool active = 16 * cw < c1 - c0;
  const __amdgpu_buffer_rsrc_t crs = make_rsrc(codes, codes_bytes);
  const __amdgpu_buffer_rsrc_t mrs = make_rsrc(meta, meta_bytes);
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(x, uint32_t(t) * uint32_t(d) * 2u);

  // the rows of slab s: a wave's i-th piece is piece `lane` of row wave + 8i
  // (zeros past t and past d), stored at position lane ^ (row & 15)
  auto xload = [&](u32x4_t (&v)[XP], int s) {
    const int k = s * kSlabCodes + 8 * lane;
#pragma unroll
    for (int i = 0; i < XP; ++i) {
      const int r = wave + 8 * i;
      v[i] = buf_load16(xrs, r < t && k < d ? (uint32_t(r) * uint32_t(d) + uint32_t(k)) * 2u : kOOB);
    }
  };
  auto xstore = [&](const u32x4_t (&v)[XP], int b) {
#pragma unroll
    for (int i = 0; i < XP; ++i) {
      const int r = wave + 8 * i;
      *reinterpret_cast<u32x4_t*>(&xs[b * XB + mr_at(r, kSlabCodes, lane)]) = v[i];
      if constexpr (AFF) {
        // the row's sum over 64-code group lane / 8: eight pieces, eight
        // lanes; a piece's pairs as bf16 dots against (1, 1)
        constexpr uint32_t kOnes = 0x3F803F80u;
        float p = dot2_bf16(v[i][3], kOnes, dot2_bf16(v[i][2], kOnes, dot2_bf16(v[i][1], kOnes, dot2_bf16(v[i][0], kOnes, 0.f))));
        p += dpp_f<0xB1>(p);    // quad_perm [1,0,3,2]
        p += dpp_f<0x4E>(p);    // quad_perm [2,3,0,1]
        p += dpp_f<0x141>(p);   // row_half_mirror
        if ((lane & 7) == 0) xsum[(b * 8 + (lane >> 3)) * XR + r] = p;
      }
    }
  };

  // the code ring: the lane's chunk of steps 2kh and 2kh + 1 of slab s and
  // the metadata of those steps (affine: dwords 4kh .. 4kh + 3, groups 4kh ..
  // 4kh + 3; MXFP4: the slab's four dwords)
  u32x4_t rc[kStRing][2];
  u32x4_t rm[kStRing];
  auto issue = [&](u32x4_t (&c2)[2], u32x4_t& m, int s) {
    const bool in = active && s < ns;
    const int w = in ? L.width(s) : 0;
    const uint32_t cb = in ? uint32_t(L.codes(s, lcol)) : 0u;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int kk = 128 * (2 * kh + j) + 32 * g;
      c2[j] = buf_load16(crs, kk < w ? cb + uint32_t(kk >> 1) : kOOB);
    }
    const int mrow = in ? L.meta_row(s) : 0;
    const uint32_t mb = in ? uint32_t(L.meta(s, lcol)) : 0u;
    const int mo = AFF ? 16 * kh : 0;
    m = buf_load16(mrs, mo < mrow ? mb + uint32_t(mo) : kOOB);
  };

  // rows of slab s in xv[s % kStXd] until stored into LDS buffer s & 1.
  // Every step issues the same loads (past the last slab they read nothing),
  // so that the compiler's count of loads in flight stays exact: a load under
  // a branch makes it wait for all of them before the next MFMA.
  u32x4_t xv[kStXd][XP];
#pragma unroll
  for (int i = 0; i < kStXd; ++i) xload(xv[i], i);
#pragma unroll
  for (int j = 0; j < kStRing; ++j) issue(rc[j], rm[j], j);
  xstore(xv[0], 0);
  __syncthreads();

  uint32_t pmask, pmagic;   // see mrow_kernel
  asm volatile("s_mov_b32 %0, 0x000f000f" : "=s"(pmask));
  asm volatile("v_mov_b32 %0, 0x43004300" : "=v"(pmagic));
  // A-operand offsets of row block 0 (row col_l) in step 0; block rb adds 16·rb
  // rows, step st 128·st elements
  int aoff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p0 = AFF ? 8 * (i >> 1) + 4 * (g & 1) + 2 + (i & 1) - 2 * (g >> 1) : 4 * g + i;
    aoff[i] = col_l * kSlabCodes + ((p0 ^ col_l) << 3);
  }
  f32x4_t acc[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) acc[rb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto slab = [&](const u32x4_t (&c2)[2], const u32x4_t& m, int s, int b) {
    const int w = L.width(s);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int st = 2 * kh + j;
      if (128 * st >= w) break;   // a narrow last slab ends early (uniform)
      const int e0 = b * XB + st * 128;   // the step's first element in row 0 of the buffer
      if constexpr (AFF) {
        const uint32_t m0 = m[2 * j];
        const uint32_t m1 = 128 * st + 64 < w ? m[2 * j + 1] : 0u;
        const float gs[2] = {bf16_lo(m0), bf16_lo(m1)};
        const float gc[2] = {__builtin_fmaf(-128.0f, bf16_lo(m0), bf16_hi(m0)),
                             __builtin_fmaf(-128.0f, bf16_lo(m1), bf16_hi(m1))};
        // each register one group in every lane (see mrow_kernel)
        const auto s20 = __builtin_amdgcn_permlane32_swap(c2[j][2], c2[j][0], false, false);
        const auto s31 = __builtin_amdgcn_permlane32_swap(c2[j][3], c2[j][1], false, false);
        const uint32_t wg[2][2] = {{s20[0], s31[0]}, {s20[1], s31[1]}};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          // the group's A operands and row sums first: one LDS wait per group
          u32x4_t a[2][RB];
          f32x4_t xg[RB];
#pragma unroll
          for (int jj = 0; jj < 2; ++jj)
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
              a[jj][rb] = *reinterpret_cast<const u32x4_t*>(&xs[aoff[2 * h + jj] + rb * 16 * kSlabCodes + e0]);
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
            xg[rb] = *reinterpret_cast<const f32x4_t*>(&xsum[(b * 8 + 2 * st + h) * XR + 16 * rb + 4 * g]);
          __builtin_amdgcn_sched_barrier(0);   // (the scheduler would interleave them one by one)
          f32x4_t pg[RB];
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) pg[rb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            u32x4_t bq;
#pragma unroll
            for (int r = 0; r < 4; ++r) bq[r] = ((wg[h][jj] >> (4 * r)) & pmask) | pmagic;
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
              pg[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a[jj][rb]),
                                                               __builtin_bit_cast(bf16x8_t, bq), pg[rb], 0, 0, 0);
          }
          // rows 16rb + 4g + r: acc += s·P + (b − 128·s)·Σx for group 2st + h
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[rb][r] = __builtin_fmaf(gc[h], xg[rb][r], __builtin_fmaf(gs[h], pg[rb][r], acc[rb][r]));
          }
        }
      } else {
        const float sc = e8m0_scale((m[st] >> (8 * g)) & 0xFFu);
#pragma unroll
        for (int hq = 0; hq < 4; hq += 2) {
          // two words' A operands first: one LDS wait per pair
          u32x4_t a[2][RB];
#pragma unroll
          for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
              a[q][rb] = *reinterpret_cast<const u32x4_t*>(&xs[aoff[hq + q] + rb * 16 * kSlabCodes + e0]);
          __builtin_amdgcn_sched_barrier(0);   // (the scheduler would interleave them one by one)
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const u32x4_t bq = mxfp4_word_to_bf16x8(c2[j][hq + q], sc);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
              acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a[q][rb]),
                                                                __builtin_bit_cast(bf16x8_t, bq), acc[rb], 0, 0, 0);
          }
        }
      }
    }
  };
  for (int s0 = 0; s0 < ns; s0 += kStRing) {
#pragma unroll
    for (int j = 0; j < kStRing; ++j) {
      const int s = s0 + j;   // s % kStXd == j % kStXd, s & 1 == j & 1
      xload(xv[j % kStXd], s + kStXd);
      if (active && s < ns) slab(rc[j], rm[j], s, j & 1);
      issue(rc[j], rm[j], s + kStRing);
      if (s + 1 < ns) xstore(xv[(j + 1) % kStXd], (j + 1) & 1);
      __syncthreads();
    }
  }

  // the second half's sums join the first's through LDS (the slab buffers
  // are free after the last barrier), then the first half stores
  f32x4_t* red = reinterpret_cast<f32x4_t*>(xs);   // [RB][4 column waves][64 lanes]
  if (kh == 1 && active) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) red[(rb * 4 + cw) * 64 + lane] = acc[rb];
  }
  __syncthreads();
  if (kh == 0 && col < c1) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const f32x4_t o = red[(rb * 4 + cw) * 64 + lane];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * rb + 4 * g + r;
        if (row < t) y[int64_t(row) * n + col] = f32_to_bf16(acc[rb][r] + o[r]);
      }
    }
  }
}

}  // namespace

int launch_mrow(const GemmArgs& a, void* stream) {
  Layout l;
  if (!layout_of(a.f, a.n, a.d, &l)) return int(hipErrorInvalidValue);
  if (!mrow_fits(a.f, a.t, a.n, a.d, l)) return int(hipErrorInvalidValue);
  hipStream_t s = static_cast<hipStream_t>(stream);
  DevInfo di{};
  const int cus = device_info(&di) == 0 && di.cus > 0 ? di.cus : 256;
  const uint8_t* codes = a.packed + l.codes_offset;
  const uint8_t* meta = a.packed + l.meta_offset;
  const uint32_t cb = uint32_t(int64_t(a.n) * (a.d / 2)), mb = uint32_t(l.meta_bytes);
  constexpr int AF = QMM_AFFINE4_G64, MX = QMM_MXFP4_G32;
  if (a.t > kMrowMaxT) {
    const MrowPlan p = mrow_stream_plan(a.n, cus);
    const dim3 grid(unsigned((a.n + p.cpw - 1) / p.cpw)), block(512);
    const size_t lds = mrow_stream_lds_bytes(a.f, a.t);
    auto go = [&](auto kern) {
      launch_kernel_lds(kern, grid, block, lds, s, codes, meta, cb, mb, a.t, a.n, a.d, p.cpw, a.x, a.y);
    };
    const int rb = mrow_stream_blocks(a.t);
    if (a.f == AF)
      rb == 2 ? go(mrow_stream_kernel<AF, 2>) : rb == 3 ? go(mrow_stream_kernel<AF, 3>) : go(mrow_stream_kernel<AF, 4>);
    else
      rb == 2 ? go(mrow_stream_kernel<MX, 2>) : rb == 3 ? go(mrow_stream_kernel<MX, 3>) : go(mrow_stream_kernel<MX, 4>);
    return int(hipGetLastError());
  }
  const MrowPlan p = mrow_plan(a.n, a.d, cus);
  const dim3 grid(unsigned((a.n + p.cpw - 1) / p.cpw)), block(unsigned(64 * p.ncw * p.kq));
  const size_t lds = mrow_lds_bytes(a.f, a.t, a.d);
  auto go = [&](auto kern) {
    launch_kernel_lds(kern, grid, block, lds, s, codes, meta, cb, mb, a.t, a.n, a.d, p.cpw, p.ncw, a.x, a.y,
                      MrowGroups{});
  };
  if (a.f == AF && a.t <= kMrowG2MaxT)
    p.kq == 4 ? go(mrow_kernel<AF, 4, true, false>) : p.kq == 2 ? go(mrow_kernel<AF, 2, true, false>)
              : go(mrow_kernel<AF, 1, true, false>);
  else if (a.f == AF)
    p.kq == 4 ? go(mrow_kernel<AF, 4, false, false>) : p.kq == 2 ? go(mrow_kernel<AF, 2, false, false>)
              : go(mrow_kernel<AF, 1, false, false>);
  else
    p.kq == 4 ? go(mrow_kernel<MX, 4, false, false>) : p.kq == 2 ? go(mrow_kernel<MX, 2, false, false>)
              : go(mrow_kernel<MX, 1, false, false>);
  return int(hipGetLastError());
}

// Grouped: 128-column workgroups (eight column waves over all slabs), one
// per (column block, segment); empty segments return at once.  Measured
// against 64 columns with two wave groups over the slabs and 32 with four:
// 128 columns 10-40% faster than either on the decode experts.
int launch_mrow_grouped(const MrowGroupedArgs& a, void* stream) {
  Layout l;
  if (!layout_of(a.f, a.n, a.d, &l)) return int(hipErrorInvalidValue);
  if (!mrow_grouped_fits(a.f, a.t, a.n, a.d, a.grp.t_x, l) || a.n_seg < 1 || a.n_seg > 65535)
    return int(hipErrorInvalidValue);
  hipStream_t s = static_cast<hipStream_t>(stream);
  constexpr int ncw = kMrowMaxWaves;
  const int cpw = a.glu ? 16 * ncw / 2 : 16 * ncw;   // output columns per workgroup
  const int nout = a.glu ? a.n / 2 : a.n;
  const dim3 grid(unsigned((nout + cpw - 1) / cpw), unsigned(a.n_seg)), block(unsigned(64 * ncw));
  const size_t lds = mrow_grouped_lds_bytes(a.f, a.t, a.d);
  const uint8_t* codes = a.stack + l.codes_offset;
  const uint8_t* meta = a.stack + l.meta_offset;
  const uint32_t cb = uint32_t(int64_t(a.n) * (a.d / 2)), mb = uint32_t(l.meta_bytes);
  auto go = [&](auto kern) {
    launch_kernel_lds(kern, grid, block, lds, s, codes, meta, cb, mb, a.t, a.n, a.d, cpw, ncw, a.x, a.y, a.grp);
  };
  constexpr int AF = QMM_AFFINE4_G64, MX = QMM_MXFP4_G32;
  if (a.glu && (a.n % 2 != 0)) return int(hipErrorInvalidValue);
  if (a.f == AF && a.t <= kMrowG2MaxT)
    a.glu ? go(mrow_kernel<AF, 1, true, true, true>) : go(mrow_kernel<AF, 1, true, true>);
  else if (a.f == AF)
    a.glu ? go(mrow_kernel<AF, 1, false, true, true>) : go(mrow_kernel<AF, 1, false, true>);
  else
    a.glu ? go(mrow_kernel<MX, 1, false, true, true>) : go(mrow_kernel<MX, 1, false, true>);
  return int(hipGetLastError());
}

}  // namespace qmm
