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

// The static scratch of qmm_gemm_noalloc (qmm_noalloc.hip): its size, and
// its device address on the device of `stream` (the current device for a
// NULL stream), looked up once per device.  0 on success, else a hipError_t.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
int noalloc_scratch(void* stream, void** out);

// The tile GEMM split along K for t > kSkinnyMaxT while its 128-row tiles
// would cover at most half of a 256-CU chip: up to kTileSplits fp32 [t][n]
// planes (whole-region weight addressing only: d a multiple of 512).  Eight
// measured 10-30% faster than four on narrow matrices (n <= 8192, 65 <= t
// <= 256, d = 5120) and within a few percent elsewhere; ten or sixteen no
// better than eight.  Where eight planes and the kernel's other regions
// (`base` bytes) would pass the allocation-free scratch, the workspace holds
// kTileSplitsWide planes instead (the earlier four), so that qmm_gemm and
// qmm_gemm_noalloc split alike wherever the latter takes the shape.
constexpr int kTileSplits = 8;
constexpr int kTileSplitsWide = 4;
inline size_t tile_split_planes_bytes(int64_t t, int64_t n, int64_t d, const Layout& l, int64_t base) {
  const bool whole = d % kSlabCodes == 0 && n * (d / 2) + (int64_t(1) << 16) < (int64_t(1) << 31) &&
                     l.meta_bytes + (int64_t(1) << 20) < (int64_t(1) << 31);
  const int64_t tiles128 = ((t + 127) / 128) * ((n + 255) / 256);
  if (!whole || t <= kSkinnyMaxT || tiles128 > 128 || d / 64 < 16 ||
      int64_t(kTileSplits) * t * n >= (int64_t(1) << 31))
    return 0;
  const int64_t plane = t * n * 4;
  const int64_t k = base + kTileSplits * plane <= int64_t(kNoAllocScratchBytes) ? kTileSplits : kTileSplitsWide;
  return size_t(k * plane);
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
  TileWs w{0, 0, 0, 0, 0};
  if (f == QMM_AFFINE4_G64) {
    w.rowe = round_up(t * d * 2, 256);
    w.colf = w.rowe + round_up(t * 4, 256);
    w.planes = w.colf + round_up(n * 4, 256);
  }
  w.total = w.planes + int64_t(tile_split_planes_bytes(t, n, d, l, w.planes));
  return w;
}

// The tile GEMM, split along K through the workspace when it helps and
// ws_bytes allows; affine weights need the workspace (tile_ws_layout), MXFP4
// weights take ws NULL (launch_gemm).
int launch_gemm_ws(const GemmArgs& a, float* ws, size_t ws_bytes, void* stream);

// y[i] = bf16(Σ_p ws[p·tn + i]) over `planes` planes in order; `stop`, when
// not NULL, is a hipEvent_t stamped by the kernel's dispatch.
void launch_partials_sum(const float* ws, int64_t tn, int planes, uint16_t* y, void* stop, void* stream);

}  // namespace qmm
