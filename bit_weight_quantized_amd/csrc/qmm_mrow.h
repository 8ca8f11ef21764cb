// Launcher of the multi-row GEMV (qmm_mrow.hip): Y = X·Ŵᵀ for a few rows,
// every weight byte read once, the rows held whole in LDS (up to 16) or
// streamed through it slab by slab (up to 64).
#pragma once

#include <stddef.h>

#include "qmm_internal.h"

namespace qmm {

constexpr int kMrowMaxT = 16;                     // rows per launch: one 16-row MFMA block
constexpr size_t kMrowMaxLds = size_t(160) << 10; // the LDS of one compute unit

constexpr int kMrowMaxWaves = 8;                  // waves per workgroup (512 threads)
constexpr size_t kMrowRedBytes = size_t(6) << 10;  // LDS for the partial sums: (kq − 1)·ncw ≤ 6 waves

// Launch shape: `groups` workgroups, a multiple of the CU count (one resident
// per CU), each taking cpw <= 128 consecutive columns with ncw column waves
// (16 columns each) times kq wave groups that share out the slabs of d, kq as
// large as 8 waves allow (and no larger than the slab count).
struct MrowPlan {
  int64_t groups;
  int cpw, ncw, kq;
};
inline MrowPlan mrow_plan(int64_t n, int64_t d, int cus) {
  const int64_t ns = (d + kSlabCodes - 1) / kSlabCodes;
  MrowPlan p;
  p.groups = (n + int64_t(cus) * 128 - 1) / (int64_t(cus) * 128) * cus;
  p.cpw = int((n + p.groups - 1) / p.groups);
  p.ncw = (p.cpw + 15) / 16;
  p.kq = ns >= 4 && 4 * p.ncw <= kMrowMaxWaves ? 4 : ns >= 2 && 2 * p.ncw <= kMrowMaxWaves ? 2 : 1;
  return p;
}

// Affine weights with at most this many rows put a step's two 64-code groups
// in the two 8-row halves of one MFMA (one row of zeros more in LDS).
constexpr int kMrowG2MaxT = 8;

// LDS of one workgroup: the t rows padded to whole 512-code slabs (bf16),
// plus a row of zeros for affine weights with t <= 8; for affine weights the
// sums of 16 rows (zeros past t) over each 64-code group (fp32); the partial
// sums of the wave groups past the first.
inline size_t mrow_lds_bytes(int f, int64_t t, int64_t d) {
  const int64_t rs = (d + kSlabCodes - 1) / kSlabCodes * kSlabCodes;
  const bool aff = f == QMM_AFFINE4_G64;
  const int64_t rows = t + (aff && t <= kMrowG2MaxT ? 1 : 0);
  return size_t(rows * rs * 2 + (aff ? (rs / 64) * 16 * 4 : 0)) + kMrowRedBytes;
}

// The streaming form, for kMrowMaxT < t <= kMrowStreamMaxT: the rows pass
// through two LDS buffers of one 512-code slab each, RB = ceil(t / 16) blocks
// of 16 rows; four waves of 16 columns per workgroup, so at most 64 columns.
constexpr int kMrowStreamMaxT = 64;
constexpr int kMrowStreamCols = 64;
inline int mrow_stream_blocks(int64_t t) { return int((t + 15) / 16); }
inline MrowPlan mrow_stream_plan(int64_t n, int cus) {
  MrowPlan p;
  p.groups = (n + int64_t(cus) * kMrowStreamCols - 1) / (int64_t(cus) * kMrowStreamCols) * cus;
  p.cpw = int((n + p.groups - 1) / p.groups);
  p.ncw = 4;
  p.kq = 1;
  return p;
}
// two slab buffers of 16·RB rows (bf16); for affine weights each buffer's
// sums of those rows over its eight 64-code groups (fp32)
inline size_t mrow_stream_lds_bytes(int f, int64_t t) {
  const int64_t rows = 16 * int64_t(mrow_stream_blocks(t));
  return size_t(2 * rows * kSlabCodes * 2 + (f == QMM_AFFINE4_G64 ? 2 * 8 * rows * 4 : 0));
}

// Whether the kernel takes this shape: 2 <= t <= 16 with the rows in LDS, or
// up to kMrowStreamMaxT rows streamed, and the 32-bit buffer offsets cover
// the codes, metadata and activations.
inline bool mrow_fits(int f, int64_t t, int64_t n, int64_t d, const Layout& l) {
  const bool shape = t >= 2 && t <= kMrowMaxT ? mrow_lds_bytes(f, t, d) <= kMrowMaxLds
                                              : t > kMrowMaxT && t <= kMrowStreamMaxT;
  return shape && n * (d / 2) < (int64_t(1) << 31) && l.meta_bytes < (int64_t(1) << 31) &&
         t * d * 2 < (int64_t(1) << 31);
}

// Y = X·Ŵᵀ for a shape mrow_fits accepts; no workspace.
int launch_mrow(const GemmArgs& a, void* stream);

// Routed experts through the in-LDS kernel: segment s's rows (gathered from
// x through row_index, or in order when it is NULL) against expert
// seg_expert[s], at most `t` rows per pass of the segment (the LDS is sized
// for t; a longer segment takes several passes).  Kernel-side view:
struct MrowGroups {
  int64_t expert_stride;        // bytes between expert blobs
  const int32_t* row_index;     // NULL: grouped row r reads x row r
  const int32_t* seg_expert;
  const int32_t* seg_offsets;
  int n_experts, m_total, t_x;
  int max_rows;                 // > 0: segments of more rows are left to another launch
};
struct MrowGroupedArgs {
  int f;
  const uint8_t* stack;         // expert 0's blob
  MrowGroups grp;
  int n_seg, t, n, d;
  const uint16_t* x;
  uint16_t* y;                  // [m_total][n], or [m_total][n/2] with glu
  bool glu;                     // y = silu(gate)·up of a gate_up stack (n even)
};
// the grouped launch's LDS: the dense one plus the chunk's x-row table
inline size_t mrow_grouped_lds_bytes(int f, int64_t t, int64_t d) {
  return mrow_lds_bytes(f, t, d) + size_t(kMrowMaxT) * 4;
}
// 2 <= t <= kMrowGroupedMaxT rows per pass within the LDS, and 32-bit
// offsets over one expert's codes and metadata and over x.  Up to 8 rows
// per segment the grouped form measured faster than the grouped matmul
// kernel on the decode experts (5-37%), at 12-16 rows not always.
constexpr int kMrowGroupedMaxT = 8;
inline bool mrow_grouped_fits(int f, int64_t t, int64_t n, int64_t d, int64_t t_x, const Layout& l) {
  return t >= 2 && t <= kMrowGroupedMaxT && mrow_grouped_lds_bytes(f, t, d) <= kMrowMaxLds &&
         n * (d / 2) < (int64_t(1) << 31) && l.meta_bytes < (int64_t(1) << 31) &&
         t_x * d * 2 < (int64_t(1) << 31);
}
int launch_mrow_grouped(const MrowGroupedArgs& a, void* stream);

// A routed call whose segments are mostly long but many short (prefill
// routing: 1 to ~60 rows per expert) splits on the device: segments of at
// most kMrowGroupedMaxT rows take the grouped multi-row kernel (max_rows),
// the others the grouped matmul kernel (skip_rows), each workgroup reading
// its segment's row count from the same tables; the two launches write
// disjoint rows of y.
int launch_grouped_gemm_long(const GemmArgs& a, int skip_rows, void* stream);

}  // namespace qmm
