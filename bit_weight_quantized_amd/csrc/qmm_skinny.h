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

// The tile GEMM split along K for t > kSkinnyMaxT while its 128-row tiles
// would cover at most half of a 256-CU chip: up to kTileSplits fp32 [t][n]
// planes (whole-region weight addressing only: d a multiple of 512).
constexpr int kTileSplits = 4;
inline size_t tile_split_planes_bytes(int64_t t, int64_t n, int64_t d, const Layout& l) {
  const bool whole = d % kSlabCodes == 0 && n * (d / 2) + (int64_t(1) << 16) < (int64_t(1) << 31) &&
                     l.meta_bytes + (int64_t(1) << 20) < (int64_t(1) << 31);
  const int64_t tiles128 = ((t + 127) / 128) * ((n + 255) / 256);
  if (!whole || t <= kSkinnyMaxT || tiles128 > 128 || d / 64 < 16 ||
      int64_t(kTileSplits) * t * n >= (int64_t(1) << 31))
    return 0;
  return size_t(kTileSplits) * size_t(t) * size_t(n) * 4;
}

// Workspace of the tile kernel.  Affine weights: the activations converted
// to fp16 (row t scaled by 2^e_t, t·d·2 bytes at `xh`), the int32 exponents
// e_t (at `rowe`) and f_c of the weight columns (at `colf`), then the K-split
// planes if the split applies (at `planes`).  MXFP4: the planes only.
// Offsets 256-byte aligned.
struct TileWs {
  int64_t xh, rowe, colf, planes, total;
};
inline TileWs tile_ws_layout(int f, int64_t t, int64_t n, int64_t d, const Layout& l) {
  const int64_t planes = int64_t(tile_split_planes_bytes(t, n, d, l));
  TileWs w{0, 0, 0, 0, planes};
  if (f == QMM_AFFINE4_G64) {
    w.rowe = round_up(t * d * 2, 256);
    w.colf = w.rowe + round_up(t * 4, 256);
    w.planes = w.colf + round_up(n * 4, 256);
    w.total = w.planes + planes;
  }
  return w;
}

// The tile GEMM, split along K through the workspace when it helps and
// ws_bytes allows; affine weights need the workspace (tile_ws_layout), MXFP4
// weights take ws NULL (launch_gemm).
int launch_gemm_ws(const GemmArgs& a, float* ws, size_t ws_bytes, void* stream);

// The static scratch of qmm_gemm_noalloc (qmm_noalloc.hip): its size, and
// its device address on the device of `stream` (the current device for a
// NULL stream), looked up once per device.  0 on success, else a hipError_t.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
int noalloc_scratch(void* stream, void** out);

// y[i] = bf16(Σ_p ws[p·tn + i]) over `planes` planes in order; `stop`, when
// not NULL, is a hipEvent_t stamped by the kernel's dispatch.
void launch_partials_sum(const float* ws, int64_t tn, int planes, uint16_t* y, void* stop, void* stream);

}  // namespace qmm
