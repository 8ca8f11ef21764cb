// Launcher of the few-row split-K GEMM (qmm_skinny.hip).  Kept apart from
// qmm_internal.h, whose contents the bf16 GEMV's recorded HBM traffic is
// keyed to.
#pragma once

#include <stddef.h>

#include "qmm_internal.h"

namespace qmm {

constexpr int kSkinnyMaxT = 64;   // rows per launch: four 16-row MFMA blocks

// fp32 partials, one [t][n] plane per 512-code slab of d
inline size_t skinny_workspace_bytes(int64_t t, int64_t n, int64_t d) {
  const int64_t slabs = (d + kSlabCodes - 1) / kSlabCodes;
  return size_t(slabs * t * n * 4);
}

// Whether the kernels' 32-bit offsets cover this shape (codes and metadata
// below 2^31 bytes, partials below 2^31 elements).
inline bool skinny_fits(int64_t t, int64_t n, int64_t d, const Layout& l) {
  return t >= 2 && t <= kSkinnyMaxT && n * (d / 2) < (int64_t(1) << 31) &&
         l.meta_bytes < (int64_t(1) << 31) &&
         int64_t(skinny_workspace_bytes(t, n, d) / 4) < (int64_t(1) << 31);
}

// Y = X·Ŵᵀ for 2 <= t <= kSkinnyMaxT rows through `ws` (skinny_workspace_bytes).
int launch_skinny(const GemmArgs& a, float* ws, void* stream);

}  // namespace qmm
