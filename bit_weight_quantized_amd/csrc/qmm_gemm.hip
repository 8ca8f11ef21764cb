// Prefill GEMM and routed-expert grouped GEMM on gfx950 MFMA.
//
// Y = X·Ŵᵀ is the one dense contraction of the path, so it runs on MFMA with
// fp32 accumulation.  Weights stay 4-bit in HBM and are dequantised in
// registers into MFMA B operands, never written back to memory (materialising
// them would move four times the bytes).  The operands are exact or rounded
// once within the tolerance: MXFP4 weights are bf16 values exactly; an affine
// weight s·q + b has up to 12 significant bits plus the bias, which bf16 (8
// bits) rounds by up to 2^-8 of its value -- more than the 2e-3 of Σ|x·w| the
// result may be off -- so the dense kernel runs affine weights as fp16 (11
// bits, 2^-11) against activations converted to fp16 exactly by a pre-pass,
// with a power of two per row and per column that keeps both in fp16's
// normal range, and the grouped kernel feeds the exact codes 128 + q and
// applies each group's scale and bias in fp32.  Activation tiles are shared by
// the four waves of a workgroup through LDS.
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
// Grouped kernel: one workgroup per (segment, 256-column tile; 128 output
// columns of gate and up each with the fused SwiGLU), rows of the
// segment gathered through row_index in blocks of 64, 16x16x32 MFMA so short
// segments waste little, K step 128.  Each expert's weight tile is read once
// per 64 routed rows.  Group metadata is loaded once per 512-code slab, one
// column per lane (16 or 32 contiguous bytes), and handed to the lanes that
// dequantise that column with ds_bpermute: loading it per K step and column
// block cost a quarter of the kernel's time in extra load instructions.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <type_traits>

#include "qmm_device.h"
#include "qmm_internal.h"
#include "qmm_launch.h"
#include "qmm_lds_copy.h"
#include "qmm_mrow.h"
#include "qmm_skinny.h"

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

// ---------------------------------------------------------------------------
// Dense GEMM
//
// Workgroup tile WM×256, wave w owns columns [64w, 64w + 64) and all WM rows,
// v_mfma_f32_32x32x16_bf16, K step 64.  Software pipeline per wave, one K
// step per stage:
//   * activations X(ks + 3) are copied global -> LDS by buffer loads with the
//     LDS destination (no registers), into one of four slots shared by the
//     workgroup;
//   * the wave's own weight codes and group metadata for step ks + 3 are
//     copied the same way into one of three per-wave slots;
//   * the weights of step ks + 1 are read back from LDS and dequantised into
//     bf16 B operands while the MFMAs of step ks run, starting two MFMA pairs
//     into the stage so the LDS reads have arrived;
//   * the A operand of each MFMA pair is read from LDS kAhead pairs ahead, and
//     the first kAhead of the next stage are read during this stage's last
//     pairs (X(ks + 1) is complete and visible by then), so a stage starts
//     its MFMAs right after the barrier.
// Each stage starts with one wait (the copies issued two stages back are
// complete: vmcnt counts in issue order and every stage issues the same
// number) and one barrier.  The stage body is written in issue order and
// pinned pair by pair, so the matrix core never waits for the VALU work.
// Rows or columns past the tile edge and k past d are out-of-range buffer
// reads and arrive as zeros, so the loop has no per-lane branches.
//
// LDS X slot: WM rows of 128 bytes (64 bf16); 16-byte chunk c of row r is
// stored at position c ^ ((r >> 1) & 7).  The LDS has 64 banks (256 bytes):
// the 16 lanes of one MFMA operand read phase touch 16 consecutive rows, and
// this swizzle puts their 16-byte pieces in 16 distinct bank groups.  The
// copies write whole 1 KiB blocks, which never conflict.
// ---------------------------------------------------------------------------

// 2^31 when k >= limit, else 0: OR-ed into a buffer offset (always below 2^31
// here) it pushes the load past every buffer range, so it returns zero.
// Arithmetic rather than a select, which the compiler would turn into
// branches around the loads.
__device__ __forceinline__ uint32_t oob_bit(int k, int limit) {
  return uint32_t(limit - 1 - k) & 0x80000000u;
}

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

// Two affine weights as fp16, each rounded once: lanes of `p` hold two codes as
// fp16 subnormals (q·2^-24 or q·2^-20, see affine_word_to_bf16x8_mix), and
// v_fma_mix{lo,hi}_f16 form fp16(sv·(fp16) + b) with the fma in fp32, so
// sv = s·2^(24 + f) (or 2^(20 + f)) and b = bias·2^f give fp16(2^f·(s·q + bias)).
// The two halves separately: a half written right after the other half of
// the same register costs a wait state, so the tile kernel issues other
// instructions between them.
__device__ __forceinline__ uint32_t mix_f16_lo(float sv, uint32_t p, float b) {
  uint32_t r;
  asm("v_fma_mixlo_f16 %0, %1, %2, %3 op_sel_hi:[0,1,0]" : "=v"(r) : "v"(sv), "v"(p), "v"(b));
  return r;
}
__device__ __forceinline__ uint32_t mix_f16_hi(uint32_t r, float sv, uint32_t p, float b) {
  asm("v_fma_mixhi_f16 %0, %1, %2, %3 op_sel:[0,1,0] op_sel_hi:[0,1,0]" : "+v"(r) : "v"(sv), "v"(p), "v"(b));
  return r;
}
__device__ __forceinline__ uint32_t mix_f16x2(float sv, uint32_t p, float b) {
  return mix_f16_hi(mix_f16_lo(sv, p, b), sv, p, b);
}

// bf16 pair r (codes 2r, 2r + 1) of an MXFP4 word; r folds to a constant
// once the caller's loops are unrolled.
__device__ __forceinline__ uint32_t mxfp4_pair(uint32_t v, float sc, int r) {
  switch (r) {
    case 0: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, sc, 0));
    case 1: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, sc, 1));
    case 2: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, sc, 2));
    default: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, sc, 3));
  }
}

// A lane's raw weights for one K step: one 16-byte chunk (32 codes) and its
// group metadata for each of its two columns.
struct WChunk {
  u32x4_t w[2];
  uint32_t m[2];
};

constexpr int kXSlots = 4;          // activation slots (copy distance 3)
constexpr int kXDist = 3;
constexpr int kWSlots = 3;          // weight slots (copy distance 3)
constexpr int kWSlotBytes = 9216;   // 256 columns × (32 B codes + 4 B metadata)

template <int WM>
constexpr int gemm_lds_bytes() {
  return kXSlots * WM * 128 + kWSlots * kWSlotBytes;
}

// Operand exponents of the affine fp16 MFMA path, one launch before the tile
// kernel.  Workgroups [0, ceil(n/64)): 64 weight columns each, f_c such that
// the column's largest |s·q + b| (at q = 0 or 15 in every group) lies in
// [2^13, 2^14), stored to col_f; lane l takes column 64·blockIdx + l and wave w
// the slabs w, w + 4, ..., three slabs' metadata in flight, and the four
// waves' maxima meet in LDS.  The following workgroups: one row of x per wave,
// scaled by 2^e_t, the power of two that puts the row's largest magnitude in
// [2^13, 2^14), converted to fp16 (xh) and e_t stored (row_e).  A bf16 value
// has 8 significant bits, so it converts exactly while its scaled magnitude
// is at least 2^-17 (fp16 subnormals step by 2^-24): every element within
// 2^-30 of its row's largest; smaller ones round to the fp16 grid.  Rows of
// up to kXhRegPieces·512 elements are loaded once, all at once, and kept in
// registers; longer rows read their remainder a second time.  The tile kernel
// forms fp16(2^f_c·w) and multiplies each output by 2^-(e_t + f_c), exactly.
constexpr int kXhRegPieces = 16;   // 16-byte pieces per lane held in registers

__device__ __forceinline__ uint32_t bf16x2_to_f16x2_scaled(uint32_t v, int e) {
  const _Float16 lo = _Float16(ldexpf(bf16_lo(v), e)), hi = _Float16(ldexpf(bf16_hi(v), e));
  return uint32_t(__builtin_bit_cast(uint16_t, lo)) | (uint32_t(__builtin_bit_cast(uint16_t, hi)) << 16);
}

__global__ __launch_bounds__(256) void xh_kernel(const uint16_t* __restrict__ x, int t, int d,
                                                 uint16_t* __restrict__ xh, int* __restrict__ row_e,
                                                 const uint8_t* __restrict__ meta, int n,
                                                 int* __restrict__ col_f) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ncb = (n + 63) / 64;
  if (int(blockIdx.x) < ncb) {
    const int c = int(blockIdx.x) * 64 + lane;
    const int cc = min(c, n - 1);   // lanes past n read a real column, store nothing
    const Slabs L{n, d, QMM_AFFINE4_G64};
    float mw = 0.f;
    // slab index clamped so every load is unconditional; slabs past the
    // wave's share, and groups a narrow slab does not have, count as zeros
    const uint8_t* mq = meta + int64_t(cc >> 2) * L.meta_quad();
    const int ns = L.count();
    for (int s0 = wave; s0 < ns; s0 += 12) {
      uint32_t v[3][kSlabCodes / 64];
#pragma unroll
      for (int u = 0; u < 3; ++u) {
        const int su = s0 + 4 * u;
        const int sl = min(su, ns - 1);
        const int ng = su < ns ? L.meta_row(sl) / 4 : 0;
        const uint32_t* mp = reinterpret_cast<const uint32_t*>(mq + 4 * int64_t(sl) * L.meta_full() + (cc & 3) * L.meta_row(sl));
#pragma unroll
        for (int gi = 0; gi < kSlabCodes / 64; ++gi) v[u][gi] = mp[min(gi, L.meta_row(sl) / 4 - 1)];
#pragma unroll
        for (int gi = 0; gi < kSlabCodes / 64; ++gi) v[u][gi] = gi < ng ? v[u][gi] : 0u;
      }
#pragma unroll
      for (int u = 0; u < 3; ++u)
#pragma unroll
        for (int gi = 0; gi < kSlabCodes / 64; ++gi) {
          const float sv = bf16_lo(v[u][gi]), bv = bf16_hi(v[u][gi]);
          mw = fmaxf(mw, fmaxf(fabsf(bv), fabsf(__builtin_fmaf(15.f, sv, bv))));
        }
    }
    __shared__ float s_mw[4][64];
    s_mw[wave][lane] = mw;
    __syncthreads();
    if (wave == 0 && c < n) {
      mw = fmaxf(fmaxf(s_mw[0][lane], s_mw[1][lane]), fmaxf(s_mw[2][lane], s_mw[3][lane]));
      int f = 0;
      if (mw > 0.f) {
        int k;
        frexpf(mw, &k);   // max in [2^(k-1), 2^k)
        f = 14 - k;
      }
      col_f[c] = f;
    }
    return;
  }
  const int64_t row = int64_t(int(blockIdx.x) - ncb) * 4 + wave;
  if (row >= t) return;   // whole waves; no barrier follows
  const u32x4_t* src = reinterpret_cast<const u32x4_t*>(x + row * d);
  u32x4_t* dst = reinterpret_cast<u32x4_t*>(xh + row * d);
  const int nc = d / 8;   // 16-byte pieces (d is a multiple of 64)
  u32x4_t v[kXhRegPieces];
#pragma unroll
  for (int i = 0; i < kXhRegPieces; ++i) {
    const int c = 64 * i + lane;
    v[i] = c < nc ? src[c] : u32x4_t{0u, 0u, 0u, 0u};
  }
  uint32_t m = 0;   // largest |x| as bf16 bits (order-preserving for |x|)
#pragma unroll
  for (int i = 0; i < kXhRegPieces; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) m = max(m, max(v[i][j] & 0x7FFFu, (v[i][j] >> 16) & 0x7FFFu));
  for (int c = 64 * kXhRegPieces + lane; c < nc; c += 64) {
    const u32x4_t w = src[c];
#pragma unroll
    for (int j = 0; j < 4; ++j) m = max(m, max(w[j] & 0x7FFFu, (w[j] >> 16) & 0x7FFFu));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = max(m, uint32_t(__shfl_xor(int(m), o)));
  int e = 0;   // all-zero rows, and rows holding inf or NaN (whose outputs are not finite), stay unscaled
  if (m != 0 && m < 0x7F80u) {
    int k;
    frexpf(__uint_as_float(m << 16), &k);   // max in [2^(k-1), 2^k)
    e = 14 - k;
  }
#pragma unroll
  for (int i = 0; i < kXhRegPieces; ++i) {
    const int c = 64 * i + lane;
    if (c < nc) {
      u32x4_t o;
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = bf16x2_to_f16x2_scaled(v[i][j], e);
      dst[c] = o;
    }
  }
  for (int c = 64 * kXhRegPieces + lane; c < nc; c += 64) {
    const u32x4_t w = src[c];
    u32x4_t o;
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = bf16x2_to_f16x2_scaled(w[j], e);
    dst[c] = o;
  }
  if (lane == 0) row_e[row] = e;
}

// FAST (d a multiple of 512, so every slab is full, and the codes and the
// metadata each below 2^31 bytes): the two weight descriptors span the whole
// codes and metadata regions for the whole kernel, each lane keeps the
// constant part of its offsets, and a step adds one scalar (or 2^31 once the
// step is past d, which reads zeros); columns past n fall past the regions or
// into other slabs' codes, which only feed output columns that are never
// stored.  Otherwise each step builds descriptors bounded to its slab and tile.
//
// SPLIT (with FAST): workgroup (tile, blockIdx.y) runs the ks_per steps from
// blockIdx.y·ks_per and writes its fp32 sums to plane blockIdx.y of ws
// ([splits][t][n]) instead of y; a second kernel adds the planes in order.  A
// compile-time switch, so the unsplit kernel keeps its step loop as it was.
template <int FMT, int WM, bool FAST, bool SPLIT = false>
__global__ __launch_bounds__(256) void gemm_kernel(const uint8_t* __restrict__ codes,
                                                   const uint8_t* __restrict__ meta, int t, int n,
                                                   int d, const uint16_t* __restrict__ x,
                                                   uint16_t* __restrict__ y, int tiles_m,
                                                   int tiles_n, uint32_t codes_bytes,
                                                   uint32_t meta_bytes, int ks_per,
                                                   float* __restrict__ ws,
                                                   const int* __restrict__ row_e,
                                                   const int* __restrict__ col_f) {
  constexpr bool AFF = FMT == QMM_AFFINE4_G64;
  constexpr int RB = WM / 32;
  constexpr int XSLOT = WM * 128;
  constexpr int WBASE = kXSlots * XSLOT;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[gemm_lds_bytes<WM>()];
  __shared__ int s_colf[AFF ? 256 : 1];   // affine: per-column exponent f
  __shared__ __attribute__((aligned(16))) int s_rowe[AFF ? WM : 4];   // affine: per-row exponent e (row_e)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col_l = lane & 31, g = lane >> 5;

  // XCD-aware tile order: consecutive workgroups are dealt round-robin to the
  // 8 XCDs; give each XCD a contiguous run of tiles, N fastest, so the
  // workgroups of one XCD share an activation strip in that XCD's L2.
  const int tiles = tiles_m * tiles_n;
  int tile = blockIdx.x;
  if ((tiles & 7) == 0) tile = (blockIdx.x & 7) * (tiles >> 3) + (blockIdx.x >> 3);
  const int tm = tile / tiles_n, tn = tile % tiles_n;
  const int m0 = tm * WM, n0 = tn * 256;
  const int rows_m = min(WM, t - m0);
  const int cols_n = min(256, n - n0);

  const Slabs L{n, d, FMT};
  const int nk_all = (d + 63) / 64;
  const int ks_base = SPLIT ? int(blockIdx.y) * ks_per : 0;   // this workgroup's first K step
  const int nk = SPLIT ? min(ks_per, nk_all - ks_base) : nk_all;   // its steps
  const uint32_t lds_base = lds_addr(lds);

  // ---- affine: the fp16 operands' exponents, from the pre-pass (xh_kernel):
  // column c's weights enter as fp16(2^f_c·w), row t's activations as
  // 2^e_t·x; the epilogue multiplies by 2^-(e_t + f_c), exactly.  Read before
  // the first LDS copy: these loads are waited for by the compiler, and none
  // may be in flight once the copies' explicit counting starts.
  if constexpr (AFF) {
    s_colf[tid] = n0 + tid < n ? col_f[n0 + tid] : 0;
    if (tid < WM) s_rowe[tid] = m0 + tid < t ? row_e[m0 + tid] : 0;
  }

  // ---- activation copies: wave instruction i moves rows 8(w + 4i) .. +7 ----
  const auto xrs = make_rsrc(x + int64_t(m0) * d, uint32_t(rows_m) * uint32_t(d) * 2u);
  // instruction rows r0 = 8(w + 4i): ((r0 + lane/8) >> 1) & 7 = (4(w & 1) + lane/16) & 7
  const int xrow = lane >> 3, xpos = lane & 7, xchunk = xpos ^ ((4 * (wave & 1) + (lane >> 4)) & 7);
  const uint32_t xlane = (uint32_t(8 * wave + xrow) * uint32_t(d) + 8u * xchunk) * 2u;
  const uint32_t xstep = 64u * uint32_t(d);  // bytes between instruction i and i + 1 (32 rows)
  auto copy_x = [&](int ks, int slot, int i) {
    const int k0 = 64 * (ks + ks_base);
    uint32_t o;
    if constexpr (FAST)   // past d: 2^31 plus at most 7 row strides, still past the range
      o = xlane + ((ks < nk ? 2u * uint32_t(k0) : 0x80000000u) + uint32_t(i) * xstep);
    else
      o = (xlane + 2u * uint32_t(k0) + uint32_t(i) * xstep) | oob_bit(k0 + 8 * xchunk, d);
    copy16_to_lds(xrs, o, lds_base + slot * XSLOT + 1024 * (wave + 4 * i));
  };

  // ---- weight copies: the wave's 64 columns, codes (2 instructions, lane ->
  // column 64w + 32cb + lane%32, 16-byte half lane/32) and one metadata dword
  // per column.  Only the wave itself reads them back, each lane the piece its
  // own copy lane moved.
  const uint32_t ccol = uint32_t(64 * wave + (lane & 31)), chalf = uint32_t(lane >> 5);
  const uint32_t mcol = uint32_t(64 * wave + lane);
  const uint32_t mquad = uint32_t(L.meta_quad());
  const int64_t meta_total = L.meta_quad() * ((int64_t(n) + 3) / 4);
  // FAST: whole-region descriptors and the lanes' constant offsets
  const auto crs_all = make_rsrc(codes, codes_bytes);
  const auto mrs_all = make_rsrc(meta, meta_bytes);
  const uint32_t slab_bytes = uint32_t(n) * uint32_t(kSlabCodes / 2);
  uint32_t vcode[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) vcode[cb] = (uint32_t(n0) + ccol + 32u * cb) * uint32_t(kSlabCodes / 2) + 16u * chalf;
  const uint32_t vmeta = ((uint32_t(n0) + mcol) >> 2) * mquad + (mcol & 3) * uint32_t(L.meta_full());
  auto copy_w = [&](int ks, int slot) {
    const uint32_t dst = lds_base + WBASE + slot * kWSlotBytes;
    if constexpr (FAST) {
      const int kg = ks + ks_base;
      const int sl = kg >> 3, j = kg & 7;   // 8 steps per slab
      const bool in = ks < nk;
      const uint32_t sc = in ? uint32_t(sl) * slab_bytes + 32u * j : 0x80000000u;
      const uint32_t mk = FMT == QMM_AFFINE4_G64 ? 4u * j : 4u * (j >> 1);
      const uint32_t sm = in ? 4u * uint32_t(sl) * uint32_t(L.meta_full()) + mk : 0x80000000u;
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) copy16_to_lds(crs_all, vcode[cb] + sc, dst + 1024 * (2 * wave + cb));
      copy4_to_lds(mrs_all, vmeta + sm, dst + 8192 + 256 * wave);
      return;
    }
    const int k0 = 64 * ks;
    const bool any = k0 < d;
    const int sl = (any ? k0 : 0) >> 9;
    const int kk = k0 & (kSlabCodes - 1);
    const uint32_t hw = uint32_t(L.width(sl) >> 1), mrow = uint32_t(L.meta_row(sl));
    // byte of this step's metadata dword within a row's slab metadata
    const int mk = FMT == QMM_AFFINE4_G64 ? 4 * (kk >> 6) : 4 * (kk >> 7);
    const auto crs = make_rsrc(codes + L.codes(sl, n0) + (kk >> 1),
                               any ? uint32_t(cols_n) * hw - uint32_t(kk >> 1) : 0u);
    // quad-major metadata: column c of the tile at (c / 4)·meta_quad + (c % 4)·mrow
    const int64_t mo = L.meta(sl, n0) + mk;
    const auto mrs = make_rsrc(meta + mo, any ? uint32_t(meta_total - mo) : 0u);
    const uint32_t koob = oob_bit(k0 + 32 * int(chalf), d);
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
      copy16_to_lds(crs, ((ccol + 32u * cb) * hw + 16u * chalf) | koob,
                    dst + 1024 * (2 * wave + cb));
    copy4_to_lds(mrs, ((mcol >> 2) * mquad + (mcol & 3) * mrow) | oob_bit(k0, d),
                 dst + 8192 + 256 * wave);
  };
  // per-stage copy instructions of one wave (the stage-start wait counts them)
  constexpr int Q = RB + 3;

  // ---- LDS reads ----
  // A operand of pair (i, j): row 32i + col_l, chunk 4g + j
  uint32_t aoff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    aoff[j] = uint32_t(col_l * 128 + (((4 * g + j) ^ ((col_l >> 1) & 7)) << 4));
  auto read_w = [&](int slot, int parity, WChunk& c) {
    const uint8_t* src = lds + WBASE + slot * kWSlotBytes;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      c.w[cb] = *reinterpret_cast<const u32x4_t*>(src + 1024 * (2 * wave + cb) + 16 * lane);
      const uint8_t* mp = src + 8192 + 256 * wave + 4 * (32 * cb + col_l);
      if (FMT == QMM_AFFINE4_G64)
        c.m[cb] = *reinterpret_cast<const uint32_t*>(mp);
      else
        c.m[cb] = mp[2 * parity + g];
    }
  };

  f32x16_t acc[RB][2];
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][cb][r] = 0.f;

  // affine: the exponent f of the lane's two columns (set after the prologue's barrier)
  int cf[2] = {0, 0};

  // The 32 B-operand registers of a step, enumerated e = 8 j + 4 cb + r
  // (word j of the chunk, column cb, fp16 (affine) or bf16 (MXFP4) pair r of
  // the word).
  auto dequant_reg = [&](const WChunk& c, const AffineMix* am, const float* sc, int e) {
    const int j = e >> 3, cb = (e >> 2) & 1, r = e & 3;
    const uint32_t v = c.w[cb][j];
    if (FMT == QMM_AFFINE4_G64) {
      const uint32_t pr = (r >= 2 ? v >> 8 : v) & ((r & 1) ? 0x00F000F0u : 0x000F000Fu);
      const float sv = (r & 1) ? am[cb].s20 : am[cb].s24;
      return mix_f16x2(sv, pr, am[cb].b);
    }
    return mxfp4_pair(v, sc[cb], r);
  };
  // affine: the masked nibble pair, multiplier and bias of register e
  auto mix_args = [&](const WChunk& c, const AffineMix* am, int e, uint32_t& pr, float& sv, float& bv) {
    const int j = e >> 3, cb = (e >> 2) & 1, r = e & 3;
    const uint32_t v = c.w[cb][j];
    pr = (r >= 2 ? v >> 8 : v) & ((r & 1) ? 0x00F000F0u : 0x000F000Fu);
    sv = (r & 1) ? am[cb].s20 : am[cb].s24;
    bv = am[cb].b;
  };
  auto consts = [&](const WChunk& c, AffineMix* am, float* sc) {
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      if (FMT == QMM_AFFINE4_G64) {
        const float sv = bf16_lo(c.m[cb]), bv = bf16_hi(c.m[cb]);
        am[cb] = {ldexpf(sv, 24 + cf[cb]), ldexpf(sv, 20 + cf[cb]), ldexpf(bv, cf[cb])};
      } else {
        sc[cb] = e8m0_scale(c.m[cb]);
      }
    }
  };

  // One pipeline stage.  Pair p issues the two MFMAs of row block p % RB and
  // word p / RB, the A read kAhead pairs later, one (or two) of the step
  // ks + 1 B registers, and in pairs 0 .. Q-1 one copy instruction each.
  constexpr int NP = 4 * RB;     // MFMA pairs per step
  constexpr int kDq = 2;         // first pair that dequantises the next step's weights
  constexpr int kAhead = 5;
  static_assert(Q <= NP, "copies must fit the pairs");
  auto stage = [&](int ks, auto parc, int xs_rd, int xs_wr, int ws_rd, int ws_wr,
                   u32x4_t bcur[2][4], u32x4_t bnext[2][4], u32x4_t apre[kAhead],
                   u32x4_t anext[kAhead]) {
    constexpr int PAR = decltype(parc)::value;   // ks & 1
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(Q));
    __syncthreads();
    WChunk wn;
    read_w(ws_rd, PAR ^ 1, wn);
    const uint8_t* ab = lds + xs_rd * XSLOT;
    const int xs_nx = (xs_rd + 1) & 3;
    u32x4_t a[NP];
#pragma unroll
    for (int p = 0; p < kAhead; ++p) a[p] = apre[p];   // read during the previous stage
    AffineMix am[2];
    float sc[2];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int i = p % RB, j = p / RB;
      // this pair's share of the next step's B registers
      const int e_lo = p >= kDq ? (p - kDq) * 32 / (NP - kDq) : 0;
      const int e_hi = p >= kDq ? (p + 1 - kDq) * 32 / (NP - kDq) : 0;
      // the weight reads issued at the stage start have two pairs to arrive
      if (p == kDq) consts(wn, am, sc);
      if constexpr (AFF) {
        // affine: the low halves ahead of the pair's MFMAs, the high halves
        // after them
#pragma unroll
        for (int e = e_lo; e < e_hi; ++e) {
          uint32_t pr;
          float sv, bv;
          mix_args(wn, am, e, pr, sv, bv);
          bnext[(e >> 2) & 1][e >> 3][e & 3] = mix_f16_lo(sv, pr, bv);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        if constexpr (AFF)
          acc[i][cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
              __builtin_bit_cast(f16x8_t, a[p]), __builtin_bit_cast(f16x8_t, bcur[cb][j]),
              acc[i][cb], 0, 0, 0);
        else
          acc[i][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8_t, a[p]), __builtin_bit_cast(bf16x8_t, bcur[cb][j]),
              acc[i][cb], 0, 0, 0);
      }
      if (p + kAhead < NP) {
        const int q = p + kAhead;
        a[q] = *reinterpret_cast<const u32x4_t*>(ab + aoff[q / RB] + 4096 * (q % RB));
      } else {
        // the first A operands of the next stage: X(ks + 1) is complete (its
        // copies are two stages old) and visible since this stage's barrier
        const int q = p + kAhead - NP;
        anext[q] = *reinterpret_cast<const u32x4_t*>(lds + xs_nx * XSLOT + aoff[q / RB] + 4096 * (q % RB));
      }
      if (p < RB) copy_x(ks + kXDist, xs_wr, p);
      if (p == RB) copy_w(ks + 3, ws_wr);
      if constexpr (AFF) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int e = e_lo; e < e_hi; ++e) {
        if constexpr (AFF) {
          uint32_t pr;
          float sv, bv;
          mix_args(wn, am, e, pr, sv, bv);
          bnext[(e >> 2) & 1][e >> 3][e & 3] = mix_f16_hi(bnext[(e >> 2) & 1][e >> 3][e & 3], sv, pr, bv);
        } else {
          bnext[(e >> 2) & 1][e >> 3][e & 3] = dequant_reg(wn, am, sc, e);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // prologue: W(0) first, then the copies a steady-state stage -2 and -1
  // would have issued, so that every stage finds the same counts in flight
#pragma unroll
  for (int i = 0; i < RB; ++i) copy_x(0, 0, i);
  copy_w(0, 0);
#pragma unroll
  for (int i = 0; i < RB; ++i) copy_x(1, 1, i);
  copy_w(1, 1);
#pragma unroll
  for (int i = 0; i < RB; ++i) copy_x(2, 2, i);
  copy_w(2, 2);
  u32x4_t ba[2][4], bb[2][4];
  u32x4_t pa[kAhead], pb[kAhead];
  {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * Q));
    __syncthreads();   // X(0) copied by every wave (and the affine exponents stored)
    if constexpr (AFF) {
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) cf[cb] = s_colf[64 * wave + 32 * cb + col_l];
    }
#pragma unroll
    for (int p = 0; p < kAhead; ++p)
      pa[p] = *reinterpret_cast<const u32x4_t*>(lds + aoff[p / RB] + 4096 * (p % RB));
    WChunk w0;
    read_w(0, 0, w0);
    AffineMix am[2];
    float sc[2];
    consts(w0, am, sc);
#pragma unroll
    for (int e = 0; e < 32; ++e) ba[(e >> 2) & 1][e >> 3][e & 3] = dequant_reg(w0, am, sc, e);
  }

  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  // X slot of step k is k % 4, W slot of step k is k % 3: stage ks reads X
  // slot ks % 4 and W slot (ks + 1) % 3, and fills X slot (ks + 3) % 4 and W
  // slot ks % 3.  An odd step count runs one extra stage past d: all its
  // loads are out of range, so it adds exact zeros (a conditional exit would
  // make the compiler copy the accumulators every iteration).
  int s0 = 0;
  for (int ks = 0; ks < nk; ks += 2) {
    const int s1 = s0 == 2 ? 0 : s0 + 1, s2 = s1 == 2 ? 0 : s1 + 1;
    stage(ks, P0{}, ks & 3, (ks + 3) & 3, s1, s0, ba, bb, pa, pb);
    stage(ks + 1, P1{}, (ks + 1) & 3, ks & 3, s2, s1, bb, ba, pb, pa);
    s0 = s2;
  }

  // epilogue: lane holds column col_l of each 32x32 block, rows 8(r/4) + 4g + r%4
  float* plane = SPLIT ? ws + int64_t(blockIdx.y) * t * n : nullptr;
#pragma unroll
  for (int i = 0; i < RB; ++i) {
    // affine: the exponents of the lane's 16 rows of this block, four
    // consecutive rows per 16-byte read, all read before the first store
    int4 re[4];
    if constexpr (AFF) {
#pragma unroll
      for (int h = 0; h < 4; ++h) re[h] = *reinterpret_cast<const int4*>(&s_rowe[32 * i + 8 * h + 4 * g]);
    }
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const int cl = 64 * wave + 32 * cb + col_l;
      if (cl >= cols_n) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rl = 32 * i + 8 * (r >> 2) + 4 * g + (r & 3);
        if (rl >= rows_m) continue;
        const int64_t at = int64_t(m0 + rl) * n + n0 + cl;
        float v = acc[i][cb][r];
        if constexpr (AFF) {
          // undo the operands' power-of-two scaling (exact)
          const int4 e4 = re[r >> 2];
          const int e = (r & 3) == 0 ? e4.x : (r & 3) == 1 ? e4.y : (r & 3) == 2 ? e4.z : e4.w;
          v = ldexpf(v, -(e + cf[cb]));
        }
        if constexpr (SPLIT)
          plane[at] = v;
        else
          y[at] = f32_to_bf16(v);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Grouped GEMM (routed experts)
// ---------------------------------------------------------------------------
constexpr int kGBM = 64;    // routed rows per pass
constexpr int kGCB = 4;     // 16-column blocks per wave
constexpr int kGCols = 4 * 16 * kGCB;   // columns per workgroup
constexpr int kGXs = 136;   // LDS row stride in bf16 for a 128-wide K step

// GLU: the weights are a gate_up stack (rows [0, n/2) the gate, [n/2, n) the
// up projection) and the output is h = silu(gate)·up, [m_total][n/2]: a
// workgroup takes 128 output columns, waves 0-1 the gate rows and waves 2-3
// the matching up rows, and after the K loop the up waves hand their fp32
// accumulators to the gate waves through LDS (the activation buffers), which
// apply the activation before the one bf16 rounding.  row_index NULL: row r
// of the grouped order reads row r of x.
// Affine weights keep per-group partial sums beside the accumulators: one
// workgroup per CU, which leaves them the whole register file.
template <int FMT, bool GLU>
__global__ __launch_bounds__(256, FMT == QMM_AFFINE4_G64 ? 1 : 2) void grouped_gemm_kernel(
    const uint8_t* __restrict__ base, int64_t expert_stride, int n_experts, int64_t codes_off,
    int64_t meta_off, int n, int d, const uint16_t* __restrict__ x, int64_t t_x,
    const int32_t* __restrict__ row_index, const int32_t* __restrict__ seg_expert,
    const int32_t* __restrict__ seg_offsets, int m_total, uint16_t* __restrict__ y, int skip_rows) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][kGBM * kGXs];
  __shared__ int32_t src_row[kGBM];
  // affine: each staged row's activation sum per 64-code group of the K step,
  // and a zero operand for the lanes outside the group an MFMA sums
  __shared__ float xsum[2][kGBM][2];
  __shared__ __attribute__((aligned(16))) uint32_t zero16[4];
  if (FMT == QMM_AFFINE4_G64 && threadIdx.x < 4) zero16[threadIdx.x] = 0u;
  static_assert(sizeof(xs) >= 2 * 16 * 64 * sizeof(f32x4_t), "the up accumulators fit the activation buffers");

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col_l = lane & 15, g = lane >> 4;
  const int s = blockIdx.y;
  const int nh = n / 2;                                   // GLU output columns
  const int n0 = blockIdx.x * (GLU ? kGCols / 2 : kGCols); // first output column of the tile
  // packed row of this wave's first column, and that column's output index
  const int wout = GLU ? n0 + 64 * (wave & 1) : n0 + 64 * wave;
  const int64_t wrow = GLU ? int64_t(wave >> 1) * nh + wout : int64_t(wout);
  const int nout = GLU ? nh : n;                           // output columns

  const int r_begin = min(max(seg_offsets[s], 0), m_total);
  const int r_end = min(max(seg_offsets[s + 1], r_begin), m_total);
  if (r_end - r_begin <= max(skip_rows, 0)) return;   // no rows, or left to the multi-row kernel
  const int e = seg_expert[s];
  const bool bad_expert = e < 0 || e >= n_experts;
  const uint8_t* blob = base + (bad_expert ? 0 : int64_t(e) * expert_stride);
  const uint8_t* codes = blob + codes_off;
  const uint8_t* meta = blob + meta_off;

  const Slabs L{n, d, FMT};
  const int nk = (d + 127) / 128;

  int64_t col[kGCB];   // packed row of column block cb
  bool col_ok[kGCB];
#pragma unroll
  for (int cb = 0; cb < kGCB; ++cb) {
    col[cb] = wrow + 16 * cb + col_l;
    col_ok[cb] = wout + 16 * cb + col_l < nout;
  }

  // activation loader: copy i of wave w covers rows 16i + 4w + (lane >> 4),
  // 16 lanes on each row's 256 contiguous bytes (chunk lane & 15); a short
  // segment's rows (< 16) are spread over all four waves
  const int xc = lane & 15;
  constexpr int MW = FMT == QMM_AFFINE4_G64 ? 8 : 4;   // metadata dwords per row per full slab
  // packed row of the column whose slab metadata lane `lane` loads (clamped
  // into the wave's half of the stack)
  const int64_t mcol = (GLU ? int64_t(wave >> 1) * nh : 0) + min(wout + lane, nout - 1);
  const __amdgpu_buffer_rsrc_t mrs =
      make_rsrc(meta, uint32_t(L.meta_quad() * ((int64_t(n) + 3) / 4)));

  for (int mb = r_begin; mb < r_end; mb += kGBM) {
    const int nrows = min(kGBM, r_end - mb);
    const int nrb = (nrows + 15) >> 4;
    if (tid < kGBM) {
      int src = -1;
      if (tid < nrows) {
        src = row_index ? row_index[mb + tid] : mb + tid;
        if (bad_expert || src < 0 || src >= t_x) src = -2;
      }
      src_row[tid] = src;
    }
    __syncthreads();
    int my_src[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) my_src[i] = src_row[16 * i + 4 * wave + (lane >> 4)];

    u32x4_t xreg[4];
    auto load_x = [&](int k0) {
      const int k = k0 + 8 * xc;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        xreg[i] = (my_src[i] >= 0 && k < d) ? load16(x + int64_t(my_src[i]) * d + k) : u32x4_t{0, 0, 0, 0};
    };
    auto store_x = [&](int buf) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * i + 4 * wave + (lane >> 4);
        *reinterpret_cast<u32x4_t*>(&xs[buf][row * kGXs + 8 * xc]) = xreg[i];
        if constexpr (FMT == QMM_AFFINE4_G64) {
          // the row's sum over each group: 8 codes per lane in order, then the
          // 8 lanes of the group (chunks 8h .. 8h + 7) in a fixed tree
          float sum = 0.f;
#pragma unroll
          for (int q = 0; q < 4; ++q) sum = (sum + bf16_lo(xreg[i][q])) + bf16_hi(xreg[i][q]);
          sum += __shfl_xor(sum, 1);
          sum += __shfl_xor(sum, 2);
          sum += __shfl_xor(sum, 4);
          if ((xc & 7) == 0) xsum[buf][row][xc >> 3] = sum;
        }
      }
    };
    auto load_w = [&](u32x4_t (&wr)[kGCB], int k0) {
      const int k = k0 + 32 * g;
#pragma unroll
      for (int cb = 0; cb < kGCB; ++cb)
        wr[cb] = (col_ok[cb] && k < d) ? load16(codes + L.code_byte(col[cb], k)) : u32x4_t{0, 0, 0, 0};
    };
    // metadata of the slab starting at code k0 for the wave's column `lane`
    uint32_t mslab[MW];
    auto load_meta = [&](int k0) {
      const int sl = k0 >> 9;
      const uint32_t off = uint32_t(L.meta(sl, mcol));
      if (L.meta_row(sl) == MW * 4) {   // full slab: 16-byte aligned
#pragma unroll
        for (int i = 0; i < MW / 4; ++i) {
          const u32x4_t v = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(mrs, int(off + 16u * i), 0, 0));
#pragma unroll
          for (int j = 0; j < 4; ++j) mslab[4 * i + j] = v[j];
        }
      } else {                          // narrow last slab: dwords (bytes past d are never used)
#pragma unroll
        for (int i = 0; i < MW; ++i) mslab[i] = __builtin_amdgcn_raw_buffer_load_b32(mrs, int(off + 4u * i), 0, 0);
      }
    };

    f32x4_t acc[4][kGCB];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int cb = 0; cb < kGCB; ++cb) acc[i][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // Two weight register slots: step s waits for W(s) and at once issues the
    // loads of step s + 1 (activations, then weights into the other slot,
    // then the metadata of a slab that opens), so the next step's latency
    // runs under this step's dequantisation, barrier and MFMAs.  Loads are
    // issued in the order they are used: X(s + 1) is stored to LDS at the end
    // of step s, W(s + 1) is consumed at the start of step s + 1.
    u32x4_t wreg[2][kGCB];
    load_x(0);
    load_w(wreg[0], 0);
    load_meta(0);
    store_x(0);
    auto gstep = [&](int ks, auto P) {
      constexpr int p = decltype(P)::value;
      const int buf = ks & 1;
      const int k0 = ks * 128;
      // this step's group metadata for each column block: dword q of the slab
      // metadata (MXFP4, byte g) or dwords 2q and 2q + 1 (affine: both groups
      // of the step), from the lane that loaded it
      const int q = ks & 3;
      uint32_t mreg[kGCB], mreg1[kGCB];
      {
        uint32_t v0, v1 = 0u;
        if constexpr (FMT == QMM_AFFINE4_G64) {
          v0 = q == 0 ? mslab[0] : q == 1 ? mslab[2] : q == 2 ? mslab[4] : mslab[6];
          v1 = q == 0 ? mslab[1] : q == 1 ? mslab[3] : q == 2 ? mslab[5] : mslab[7];
        } else {
          v0 = q == 0 ? mslab[0] : q == 1 ? mslab[1] : q == 2 ? mslab[2] : mslab[3];
        }
#pragma unroll
        for (int cb = 0; cb < kGCB; ++cb) {
          const int src = 4 * (16 * cb + col_l);
          if (FMT == QMM_AFFINE4_G64) {
            mreg[cb] = uint32_t(__builtin_amdgcn_ds_bpermute(src, int(v0)));
            mreg1[cb] = uint32_t(__builtin_amdgcn_ds_bpermute(src, int(v1)));
          } else {
            mreg[cb] = (uint32_t(__builtin_amdgcn_ds_bpermute(src, int(v0))) >> (8 * g)) & 0xFFu;
          }
        }
      }
      // W(s) has arrived (its metadata with it): start step s + 1's loads
      // before the dequantisation
      if (ks + 1 < nk) {
        load_x(k0 + 128);
        load_w(wreg[p ^ 1], k0 + 128);
        if (((k0 + 128) & (kSlabCodes - 1)) == 0) load_meta(k0 + 128);
      }
      // No masking: past d the activations are zero and the weights finite
      // (affine scale and bias and E8M0 < 255 are checked at pack time), so
      // those products are exact zeros; columns past n are never stored.
      if constexpr (FMT == QMM_AFFINE4_G64) {
        // Affine: the codes enter the MFMAs as the exact bf16 values 128 + q
        // and scale and bias follow per group in fp32,
        //   Σ_k x·(s·q + b) = s·Σ_k x·(128 + q) + (b − 128·s)·Σ_k x,
        // so no weight is rounded.  Lane group g's chunk lies in group g / 2
        // of the step; the MFMAs of group h take the zero operand on the
        // other lanes, so each sums one group only.
        u32x4_t bq[4][kGCB];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int cb = 0; cb < kGCB; ++cb)
#pragma unroll
            for (int r = 0; r < 4; ++r) bq[j][cb][r] = and_or(wreg[p][cb][j] >> (4 * r), 0x000F000Fu, kMagic128x2);
        float gsc[kGCB][2], gcb[kGCB][2];   // scale and b − 128·s of the step's two groups
#pragma unroll
        for (int cb = 0; cb < kGCB; ++cb) {
          gsc[cb][0] = bf16_lo(mreg[cb]);
          gcb[cb][0] = __builtin_fmaf(-128.0f, bf16_lo(mreg[cb]), bf16_hi(mreg[cb]));
          gsc[cb][1] = bf16_lo(mreg1[cb]);
          gcb[cb][1] = __builtin_fmaf(-128.0f, bf16_lo(mreg1[cb]), bf16_hi(mreg1[cb]));
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (i < nrb) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              f32x4_t pg[kGCB];
#pragma unroll
              for (int cb = 0; cb < kGCB; ++cb) pg[cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const u32x4_t* ap = (g >> 1) == h
                                        ? reinterpret_cast<const u32x4_t*>(&xs[buf][(16 * i + col_l) * kGXs + 32 * g + 8 * j])
                                        : reinterpret_cast<const u32x4_t*>(zero16);
                const u32x4_t a = *ap;
#pragma unroll
                for (int cb = 0; cb < kGCB; ++cb)
                  pg[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                      __builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, bq[j][cb]), pg[cb], 0, 0, 0);
              }
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const float xg = xsum[buf][16 * i + 4 * g + r][h];
#pragma unroll
                for (int cb = 0; cb < kGCB; ++cb)
                  acc[i][cb][r] = __builtin_fmaf(gcb[cb][h], xg, __builtin_fmaf(gsc[cb][h], pg[cb][r], acc[i][cb][r]));
              }
            }
          }
        }
        if (ks + 1 < nk) store_x(buf ^ 1);
        return;
      }
      u32x4_t bfrag[kGCB][4];
#pragma unroll
      for (int cb = 0; cb < kGCB; ++cb) dequant_chunk<FMT>(wreg[p][cb], mreg[cb], bfrag[cb]);
      __syncthreads();
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (i < nrb) {
            const u32x4_t a = *reinterpret_cast<const u32x4_t*>(&xs[buf][(16 * i + col_l) * kGXs + 32 * g + 8 * j]);
#pragma unroll
            for (int cb = 0; cb < kGCB; ++cb)
              acc[i][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  __builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, bfrag[cb][j]),
                  acc[i][cb], 0, 0, 0);
          }
        }
      }
      if (ks + 1 < nk) store_x(buf ^ 1);
    };
    for (int ks = 0; ks < nk; ks += 2) {
      gstep(ks, std::integral_constant<int, 0>{});
      if (ks + 1 < nk) gstep(ks + 1, std::integral_constant<int, 1>{});
    }

    // epilogue: lane holds column col_l, rows 4g + r of each 16x16 block
    if (GLU) {
      f32x4_t* up = reinterpret_cast<f32x4_t*>(&xs[0][0]);   // [wave - 2][i][cb][lane]
      __syncthreads();   // every wave is done reading the activation buffers
      if (wave >= 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int cb = 0; cb < kGCB; ++cb) up[((wave - 2) * 16 + 4 * i + cb) * 64 + lane] = acc[i][cb];
      }
      __syncthreads();
      if (wave < 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (i >= nrb) continue;
#pragma unroll
          for (int cb = 0; cb < kGCB; ++cb) {
            if (!col_ok[cb]) continue;
            const f32x4_t u = up[(wave * 16 + 4 * i + cb) * 64 + lane];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int lr = 16 * i + 4 * g + r;
              if (lr < nrows) {
                const float gv = acc[i][cb][r];
                const float h = gv / (1.0f + expf(-gv)) * u[r];
                const float v = src_row[lr] == -2 ? __builtin_nanf("") : h;
                y[int64_t(mb + lr) * nh + wout + 16 * cb + col_l] = f32_to_bf16(v);
              }
            }
          }
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i >= nrb) continue;
#pragma unroll
        for (int cb = 0; cb < kGCB; ++cb) {
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
    }
    __syncthreads();  // src_row and xs are reused by the next pass
  }
}

}  // namespace

int launch_gemm(const GemmArgs& a, void* stream) { return launch_gemm_ws(a, nullptr, 0, stream); }

int launch_gemm_ws(const GemmArgs& a, float* ws, size_t ws_bytes, void* stream) {
  Layout l;
  if (!layout_of(a.f, a.n, a.d, &l)) return int(hipErrorInvalidValue);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool aff = a.f == QMM_AFFINE4_G64;
  const uint8_t* codes = a.packed + l.codes_offset;
  const uint8_t* meta = a.packed + l.meta_offset;
  const int tiles_n = (a.n + 255) / 256;
  // whole-region descriptors: offsets up to a region plus one 256-column
  // tile past it, and 2^31 as the out-of-range marker, must fit in 32 bits
  const int64_t code_bytes = int64_t(a.n) * (a.d / 2);
  const bool fast = a.d % kSlabCodes == 0 && code_bytes + (int64_t(1) << 16) < (int64_t(1) << 31) &&
                    l.meta_bytes + (int64_t(1) << 20) < (int64_t(1) << 31);
  const uint32_t cb = fast ? uint32_t(code_bytes) : 0u, mb = fast ? uint32_t(l.meta_bytes) : 0u;
  DevInfo di{};
  const int64_t cus = device_info(&di) == 0 && di.cus > 0 ? di.cus : 256;
  const int nk = (a.d + 63) / 64;
  // affine: the fp16 activations and row exponents live in the workspace,
  // the K-split planes (if any) after them
  const TileWs tw = tile_ws_layout(a.f, a.t, a.n, a.d, l);
  if (aff && (!ws || int64_t(ws_bytes) < tw.planes)) return int(hipErrorInvalidValue);
  uint8_t* wsb = reinterpret_cast<uint8_t*>(ws);
  const uint16_t* xk = aff ? reinterpret_cast<const uint16_t*>(wsb + tw.xh) : a.x;
  int* row_e = aff ? reinterpret_cast<int*>(wsb + tw.rowe) : nullptr;
  int* col_f = aff ? reinterpret_cast<int*>(wsb + tw.colf) : nullptr;
  float* planes = ws ? reinterpret_cast<float*>(wsb + tw.planes) : nullptr;
  const size_t planes_bytes = ws ? ws_bytes - size_t(tw.planes) : 0;
  ProfileEvents pe = take_profile_events();   // start with the first kernel, stop with the last
  if (aff) {
    const dim3 pgrid(unsigned((a.n + 63) / 64 + (a.t + 3) / 4));
    uint16_t* xh = reinterpret_cast<uint16_t*>(wsb + tw.xh);
    if (pe.start)
      hipExtLaunchKernelGGL(xh_kernel, pgrid, dim3(256), 0, s, static_cast<hipEvent_t>(pe.start), nullptr, 0,
                            a.x, a.t, a.d, xh, row_e, meta, a.n, col_f);
    else
      hipLaunchKernelGGL(xh_kernel, pgrid, dim3(256), 0, s, a.x, a.t, a.d, xh, row_e, meta, a.n, col_f);
    pe.start = nullptr;
  }
  auto go = [&](auto kernel, auto split_kernel, int wm) {
    const int tiles_m = (a.t + wm - 1) / wm;
    const int tiles = tiles_m * tiles_n;
    // split along K while the tiles cannot fill the chip (few rows): as many
    // splits as fit the CUs, each at least 8 steps, and no more than the
    // planes the workspace layout reserves for the shape (whatever the size of
    // the buffer passed, so the split, and with it every output bit, depends
    // on the shape only); none if the buffer holds fewer
    int splits = 1;
    if (fast && planes && a.t > kSkinnyMaxT) {
      const size_t plane = size_t(a.t) * size_t(a.n) * 4;
      const int64_t reserved = (tw.total - tw.planes) / int64_t(plane);
      splits = int(std::min<int64_t>({reserved, cus / tiles, int64_t(nk / 8)}));
      if (splits < 2 || size_t(splits) * plane > planes_bytes) splits = 1;
    }
    if (splits == 1) {
      if (pe.start || pe.stop)
        hipExtLaunchKernelGGL(kernel, dim3(unsigned(tiles)), dim3(256), 0, s,
                              static_cast<hipEvent_t>(pe.start), static_cast<hipEvent_t>(pe.stop), 0,
                              codes, meta, a.t, a.n, a.d, xk, a.y, tiles_m, tiles_n, cb, mb, nk,
                              static_cast<float*>(nullptr), static_cast<const int*>(row_e),
                              static_cast<const int*>(col_f));
      else
        hipLaunchKernelGGL(kernel, dim3(unsigned(tiles)), dim3(256), 0, s, codes, meta, a.t, a.n, a.d,
                           xk, a.y, tiles_m, tiles_n, cb, mb, nk, static_cast<float*>(nullptr),
                           static_cast<const int*>(row_e), static_cast<const int*>(col_f));
      return;
    }
    const int ks_per = (nk + splits - 1) / splits;
    splits = (nk + ks_per - 1) / ks_per;
    if (pe.start)
      hipExtLaunchKernelGGL(split_kernel, dim3(unsigned(tiles), unsigned(splits)), dim3(256), 0, s,
                            static_cast<hipEvent_t>(pe.start), nullptr, 0, codes, meta, a.t, a.n, a.d,
                            xk, a.y, tiles_m, tiles_n, cb, mb, ks_per, planes,
                            static_cast<const int*>(row_e), static_cast<const int*>(col_f));
    else
      hipLaunchKernelGGL(split_kernel, dim3(unsigned(tiles), unsigned(splits)), dim3(256), 0, s, codes, meta,
                         a.t, a.n, a.d, xk, a.y, tiles_m, tiles_n, cb, mb, ks_per, planes,
                         static_cast<const int*>(row_e), static_cast<const int*>(col_f));
    launch_partials_sum(planes, int64_t(a.t) * a.n, splits, a.y, pe.stop, s);
  };
  // Tile height by a cost model of whole rounds of tiles over the CUs: a round
  // of 256-row tiles (one per CU) takes ~12 units, a round of 128-row tiles
  // (per CU, whether one or two share it) ~7 (measured at n = 13824, d = 5120:
  // ~125 and ~73 µs).  So t = 256 / 512 run on 128-row tiles (68 / 81 µs
  // against 107 / 113), t = 768..1024 and 2048 on 256-row tiles, t = 1280..1536
  // on 128-row tiles again (225 / 232 µs against 242 / 246, where 256-row tiles
  // spill into a second round).  Each output sums its k in the same order on
  // both, so results are identical.
  const int64_t r128 = (int64_t((a.t + 127) / 128) * tiles_n + cus - 1) / cus;
  const int64_t r256 = (int64_t((a.t + 255) / 256) * tiles_n + cus - 1) / cus;
  const bool small = a.t <= 128 || 7 * r128 < 12 * r256;
  // the split kernel exists for whole-region addressing only; otherwise the
  // unsplit one is passed twice (go never splits without FAST)
  if (!small) {
    if (aff)
      fast ? go(gemm_kernel<QMM_AFFINE4_G64, 256, true>, gemm_kernel<QMM_AFFINE4_G64, 256, true, true>, 256)
           : go(gemm_kernel<QMM_AFFINE4_G64, 256, false>, gemm_kernel<QMM_AFFINE4_G64, 256, false>, 256);
    else
      fast ? go(gemm_kernel<QMM_MXFP4_G32, 256, true>, gemm_kernel<QMM_MXFP4_G32, 256, true, true>, 256)
           : go(gemm_kernel<QMM_MXFP4_G32, 256, false>, gemm_kernel<QMM_MXFP4_G32, 256, false>, 256);
  } else {
    if (aff)
      fast ? go(gemm_kernel<QMM_AFFINE4_G64, 128, true>, gemm_kernel<QMM_AFFINE4_G64, 128, true, true>, 128)
           : go(gemm_kernel<QMM_AFFINE4_G64, 128, false>, gemm_kernel<QMM_AFFINE4_G64, 128, false>, 128);
    else
      fast ? go(gemm_kernel<QMM_MXFP4_G32, 128, true>, gemm_kernel<QMM_MXFP4_G32, 128, true, true>, 128)
           : go(gemm_kernel<QMM_MXFP4_G32, 128, false>, gemm_kernel<QMM_MXFP4_G32, 128, false>, 128);
  }
  return int(hipGetLastError());
}

int launch_grouped_gemm(const GemmArgs& a, void* stream) { return launch_grouped_gemm_long(a, 0, stream); }

int launch_grouped_gemm_long(const GemmArgs& a, int skip_rows, void* stream) {
  Layout l;
  if (!layout_of(a.f, a.n, a.d, &l)) return int(hipErrorInvalidValue);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int per_tile = a.swiglu ? kGCols / 2 : kGCols;
  const int64_t outs = a.swiglu ? a.n / 2 : a.n;
  dim3 grid(unsigned((outs + per_tile - 1) / per_tile), unsigned(a.n_seg));
  auto go = [&](auto kernel) {
    launch_kernel(kernel, grid, dim3(256), s, a.packed, a.expert_stride, a.n_experts, l.codes_offset,
                  l.meta_offset, a.n, a.d, a.x, a.t_x, a.row_index, a.seg_expert, a.seg_offsets,
                  a.m_total, a.y, skip_rows);
  };
  if (a.f == QMM_AFFINE4_G64)
    a.swiglu ? go(grouped_gemm_kernel<QMM_AFFINE4_G64, true>) : go(grouped_gemm_kernel<QMM_AFFINE4_G64, false>);
  else
    a.swiglu ? go(grouped_gemm_kernel<QMM_MXFP4_G32, true>) : go(grouped_gemm_kernel<QMM_MXFP4_G32, false>);
  return int(hipGetLastError());
}

}  // namespace qmm
