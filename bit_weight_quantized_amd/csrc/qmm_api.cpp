// C-ABI entry points of libqmm: argument validation (host only, before any
// HIP call), kernel selection and error mapping.  See include/qmm.h.
#include <hip/hip_runtime.h>

#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "qmm_deferred.h"
#include "qmm_internal.h"
#include "qmm_mrow.h"
#include "qmm_skinny.h"

namespace {

thread_local char g_last_error[256] = "";
thread_local qmm::ProfileEvents g_profile = {nullptr, nullptr};

qmm_status fail(qmm_status s, const char* what) {
  snprintf(g_last_error, sizeof(g_last_error), "%s", what);
  return s;
}

qmm_status hip_fail(int err, const char* where) {
  snprintf(g_last_error, sizeof(g_last_error), "%s: %s", where,
           hipGetErrorString(static_cast<hipError_t>(err)));
  return QMM_E_HIP;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool valid_format(int f) { return f == QMM_AFFINE4_G64 || f == QMM_MXFP4_G32; }

qmm_status check_shape(int f, int64_t n, int64_t d, qmm::Layout* l) {
  if (!valid_format(f)) return fail(QMM_E_ARG, "unknown format");
  if (n < 1 || d < 1) return fail(QMM_E_ARG, "n and d must be >= 1");
  if (!qmm::layout_of(f, n, d, l)) return fail(QMM_E_SHAPE, "d must be a multiple of the group size, n <= 2^28, d <= 65536");
  return QMM_OK;
}

// The GEMV kernels address one matrix's codes and metadata through 32-bit
// buffer offsets, with 2^31 reserved as the out-of-range marker.
bool gemv_fits(int64_t n, int64_t d, const qmm::Layout& l) {
  return n * (d / 2) < (int64_t(1) << 31) && l.meta_bytes < (int64_t(1) << 31);
}

// A workspace is optional; one that is passed must hold what the call uses.
qmm_status check_ws(size_t need, const void* ws, size_t ws_bytes) {
  if (ws && ws_bytes < need) return fail(QMM_E_WORKSPACE, "workspace smaller than qmm_workspace_bytes()");
  return QMM_OK;
}

// Kernel override (qmm_set_kernel / QMM_FORCE_KERNEL): process-wide.
constexpr int kKernelUnset = -2, kKernelInvalid = -1;
std::atomic<int> g_kernel{kKernelUnset};

int parse_kernel(const char* v) {
  if (!v || !*v || !strcmp(v, "auto") || !strcmp(v, "0")) return QMM_KERNEL_AUTO;
  if (!strcmp(v, "tile") || !strcmp(v, "1")) return QMM_KERNEL_TILE;
  if (!strcmp(v, "tile_unsplit") || !strcmp(v, "2")) return QMM_KERNEL_TILE_UNSPLIT;
  if (!strcmp(v, "few_row") || !strcmp(v, "3")) return QMM_KERNEL_FEW_ROW;
  if (!strcmp(v, "grouped_matmul") || !strcmp(v, "4")) return QMM_KERNEL_GROUPED_MATMUL;
  if (!strcmp(v, "multi_row") || !strcmp(v, "5")) return QMM_KERNEL_MULTI_ROW;
  return kKernelInvalid;
}

// The environment is read once, at the first use; qmm_set_kernel wins over it.
int forced_kernel() {
  static std::once_flag once;
  std::call_once(once, [] {
    int unset = kKernelUnset;
    g_kernel.compare_exchange_strong(unset, parse_kernel(getenv("QMM_FORCE_KERNEL")));
  });
  return g_kernel.load(std::memory_order_relaxed);
}

qmm_status check_kernel(int* k) {
  *k = forced_kernel();
  if (*k == kKernelInvalid)
    return fail(QMM_E_ARG, "QMM_FORCE_KERNEL is not one of auto, tile, tile_unsplit, few_row, grouped_matmul, multi_row (or 0..5)");
  return QMM_OK;
}

bool forces_tile(int k) { return k == QMM_KERNEL_TILE || k == QMM_KERNEL_TILE_UNSPLIT; }

// Whether qmm_gemm runs the multi-row GEMV under kernel setting k: when
// forced, or by default where it was measured faster than the few-row
// split-K kernel.  Each of its workgroups stages every activation row, so
// narrow matrices (few columns per workgroup) favour the split-K kernel.
// Rows held in LDS (t <= 16): wherever d <= 3072 (a short reduction leaves
// the split-K kernel little to share out beside its second launch), else
// MXFP4 weights from 5120 columns, or for up to 8 rows, and affine weights,
// whose per-group scale and bias cost more per code, from 8192.  Rows streamed (17 <= t <= 64): wherever d <= 2048 (the
// split-K kernel then has few slabs to share out), else from 6912 columns
// while d <= 5120 and from 10240 beyond (below those the split-K grid fits
// about one round of workgroups and wins).
bool uses_mrow(int k, int f, int64_t t, int64_t n, int64_t d, const qmm::Layout& l) {
  if (k == QMM_KERNEL_MULTI_ROW) return qmm::mrow_fits(f, t, n, d, l);
  // (the grouped-matmul setting does not concern qmm_gemm: as under auto)
  if ((k != QMM_KERNEL_AUTO && k != QMM_KERNEL_GROUPED_MATMUL) || !qmm::mrow_fits(f, t, n, d, l)) return false;
  if (t > qmm::kMrowMaxT) return d <= 2048 || (n >= 6912 && d <= 5120) || n >= 10240;
  if (d <= 3072) return true;
  return f == QMM_MXFP4_G32 ? (n >= 5120 || t <= 8) : n >= 8192;
}

// Workspace of qmm_gemm under kernel setting k (0 where the call runs no
// kernel that takes one, or where it fails).
size_t gemm_ws_bytes(int k, int f, int64_t t, int64_t n, int64_t d, const qmm::Layout& l) {
  if (t < 1 || t > qmm::kMaxT) return 0;
  if (forces_tile(k)) {
    const qmm::TileWs tw = qmm::tile_ws_layout(f, t, n, d, l);
    return size_t(k == QMM_KERNEL_TILE_UNSPLIT ? tw.planes : tw.total);
  }
  if (t < 2) return 0;
  if (k == QMM_KERNEL_FEW_ROW) return qmm::skinny_fits(t, n, d, l) ? qmm::skinny_workspace_bytes(t, n, d) : 0;
  if (k == QMM_KERNEL_MULTI_ROW || uses_mrow(k, f, t, n, d, l)) return 0;
  return qmm::skinny_fits(t, n, d, l) ? qmm::skinny_workspace_bytes(t, n, d)
                                      : size_t(qmm::tile_ws_layout(f, t, n, d, l).total);
}

}  // namespace

qmm::ProfileEvents qmm::take_profile_events() {
  const ProfileEvents pe = g_profile;
  g_profile = {nullptr, nullptr};
  return pe;
}

extern "C" {

qmm_status qmm_profile_next(void* start_event, void* stop_event) {
  g_profile = {start_event, stop_event};
  return QMM_OK;
}

size_t qmm_packed_bytes(qmm_format f, int64_t n, int64_t d) {
  qmm::Layout l;
  if (!valid_format(f) || !qmm::layout_of(f, n, d, &l)) return 0;
  return size_t(l.total_bytes);
}

size_t qmm_workspace_bytes(qmm_format f, int64_t t, int64_t n, int64_t d) {
  qmm::Layout l;
  if (!valid_format(f) || n < 1 || d < 1 || !qmm::layout_of(f, n, d, &l)) return 0;
  const int k = forced_kernel();
  return k == kKernelInvalid ? 0 : gemm_ws_bytes(k, f, t, n, d, l);
}

qmm_status qmm_set_kernel(qmm_kernel k) {
  g_last_error[0] = 0;
  if (k < QMM_KERNEL_AUTO || k > QMM_KERNEL_MULTI_ROW) return fail(QMM_E_ARG, "unknown kernel setting");
  forced_kernel();   // the environment is consumed first, so it cannot override this later
  g_kernel.store(int(k), std::memory_order_relaxed);
  return QMM_OK;
}

int qmm_get_kernel(void) { return forced_kernel(); }

uint32_t qmm_layout_version(void) { return qmm::kLayoutVersion; }

qmm_status qmm_route(const qmm_bf16* x, int64_t t, int64_t d, const qmm_bf16* r, int32_t n_experts,
                     const float* bias, int32_t k, float* scores, int32_t* topk,
                     int32_t* seg_expert, int32_t* seg_offsets, int32_t* row_index, void* stream) {
  g_last_error[0] = 0;
  if (!x || !r || !scores || !topk || !seg_expert || !seg_offsets || !row_index)
    return fail(QMM_E_ARG, "NULL pointer");
  if (t < 1 || n_experts < 1 || k < 1) return fail(QMM_E_ARG, "t, n_experts and k must be >= 1");
  if (n_experts > qmm::kRouteMaxExperts) return fail(QMM_E_SHAPE, "n_experts must be <= 1024");
  if (k > qmm::kRouteMaxK || k > n_experts) return fail(QMM_E_SHAPE, "k must be <= min(64, n_experts)");
  if (d < 8 || d % 8 || d > qmm::kMaxD) return fail(QMM_E_SHAPE, "d must be a multiple of 8 in [8, 65536]");
  if (t * d * 2 >= (int64_t(1) << 31) || int64_t(n_experts) * d * 2 >= (int64_t(1) << 31))
    return fail(QMM_E_SHAPE, "x and r must each be under 2 GiB");
  if (t * k >= (int64_t(1) << 30)) return fail(QMM_E_SHAPE, "t*k must be below 2^30");
  if (!aligned(x, 16) || !aligned(r, 16)) return fail(QMM_E_ALIGN, "x and r must be 16-byte aligned");
  if (!aligned(scores, 4) || !aligned(topk, 4) || !aligned(seg_expert, 4) || !aligned(seg_offsets, 4) ||
      !aligned(row_index, 4) || (bias && !aligned(bias, 4)))
    return fail(QMM_E_ALIGN, "scores, bias and the tables must be 4-byte aligned");
  qmm::RouteArgs a{x, int(t), int(d), r, n_experts, bias, k, scores, topk, seg_expert, seg_offsets, row_index};
  int err = qmm::launch_route(a, stream);
  if (err) return hip_fail(err, "qmm_route");
  return QMM_OK;
}

qmm_status qmm_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  g_last_error[0] = 0;
  if (!src || !sink) return fail(QMM_E_ARG, "NULL pointer");
  if (!aligned(src, 16) || !aligned(sink, 4)) return fail(QMM_E_ALIGN, "src must be 16-byte, sink 4-byte aligned");
  if (bytes == 0 || bytes % 16 || bytes >= (size_t(1) << 31))
    return fail(QMM_E_SHAPE, "bytes must be a positive multiple of 16 below 2^31");
  int err = qmm::launch_stream_read(src, bytes, sink, stream);
  if (err) return hip_fail(err, "qmm_stream_read");
  return QMM_OK;
}

const char* qmm_last_error(void) { return g_last_error; }

const char* qmm_status_string(qmm_status s) {
  switch (s) {
    case QMM_OK: return "ok";
    case QMM_E_ARG: return "invalid argument";
    case QMM_E_SHAPE: return "unsupported shape";
    case QMM_E_ALIGN: return "misaligned pointer";
    case QMM_E_UNSUPPORTED: return "unsupported request";
    case QMM_E_WORKSPACE: return "workspace too small";
    case QMM_E_HIP: return "HIP runtime error";
    case QMM_E_LAYOUT: return "packed blob does not match the requested weights";
    case QMM_E_VALUE: return "value outside the format";
  }
  return "unknown status";
}

qmm_status qmm_pack(qmm_format f, int64_t n, int64_t d, const void* codes, const void* scales,
                    const void* biases, void* packed, void* stream) {
  g_last_error[0] = 0;
  qmm::Layout l;
  qmm_status st = check_shape(f, n, d, &l);
  if (st) return st;
  if (!codes || !scales || !packed) return fail(QMM_E_ARG, "NULL pointer");
  if (f == QMM_AFFINE4_G64 && !biases) return fail(QMM_E_ARG, "affine weights need biases");
  if (f == QMM_MXFP4_G32 && biases) return fail(QMM_E_ARG, "MXFP4 weights take no biases");
  if (!aligned(packed, 256)) return fail(QMM_E_ALIGN, "packed must be 256-byte aligned");
  if (!aligned(codes, 4) || !aligned(scales, 2) || (biases && !aligned(biases, 2)))
    return fail(QMM_E_ALIGN, "codes must be 4-byte, scales/biases 2-byte aligned");
  int err = qmm::launch_pack(f, n, d, codes, scales, biases, packed, stream);
  if (err) return hip_fail(err, "qmm_pack");
  qmm::PackedHeader h;
  err = qmm::read_header(packed, &h, stream);
  if (err) return hip_fail(err, "qmm_pack");
  if (h.flags & qmm::kFlagInvalid)
    return fail(QMM_E_VALUE, f == QMM_MXFP4_G32
                                 ? "E8M0 scale 255 (NaN) in the input"
                                 : "affine scale not finite or |scale| >= 2^100, or bias not finite");
  return QMM_OK;
}

qmm_status qmm_unpack(qmm_format f, int64_t n, int64_t d, const void* packed, void* codes,
                      void* scales, void* biases, void* stream) {
  g_last_error[0] = 0;
  qmm::Layout l;
  qmm_status st = check_shape(f, n, d, &l);
  if (st) return st;
  if (!codes || !scales || !packed) return fail(QMM_E_ARG, "NULL pointer");
  if (f == QMM_AFFINE4_G64 && !biases) return fail(QMM_E_ARG, "affine weights need biases");
  if (!aligned(packed, 256)) return fail(QMM_E_ALIGN, "packed must be 256-byte aligned");
  if (!aligned(codes, 4) || !aligned(scales, 2) || (biases && !aligned(biases, 2)))
    return fail(QMM_E_ALIGN, "codes must be 4-byte, scales/biases 2-byte aligned");
  qmm::PackedHeader h;
  int err = qmm::read_header(packed, &h, stream);
  if (err) return hip_fail(err, "qmm_unpack");
  if (h.magic != qmm::kMagic || h.version != qmm::kLayoutVersion || h.format != uint32_t(f) ||
      h.n != n || h.d != d || (h.flags & qmm::kFlagInvalid))
    return fail(QMM_E_LAYOUT, "blob header does not match (magic, version, format, n, d)");
  err = qmm::launch_unpack(f, n, d, packed, codes, scales, biases, stream);
  if (err) return hip_fail(err, "qmm_unpack");
  return QMM_OK;
}

qmm_status qmm_gemv(qmm_format f, const void* packed, int64_t n, int64_t d, const qmm_bf16* x,
                    qmm_bf16* y, void* ws, size_t ws_bytes, void* stream) {
  g_last_error[0] = 0;
  qmm::Layout l;
  qmm_status st = check_shape(f, n, d, &l);
  if (st) return st;
  if (!gemv_fits(n, d, l)) return fail(QMM_E_SHAPE, "the GEMV addresses codes and metadata with 32-bit offsets: n*d/2 must be below 2^31");
  if (!packed || !x || !y) return fail(QMM_E_ARG, "NULL pointer");
  if (!aligned(packed, 256)) return fail(QMM_E_ALIGN, "packed must be 256-byte aligned");
  if (!aligned(x, 16)) return fail(QMM_E_ALIGN, "x must be 16-byte aligned");
  if (!aligned(y, 2)) return fail(QMM_E_ALIGN, "y must be 2-byte aligned");
  if ((st = check_ws(0, ws, ws_bytes))) return st;
  qmm::GemvArgs a{};
  a.f = f;
  a.packed = static_cast<const uint8_t*>(packed);
  a.n = int(n);
  a.d = int(d);
  a.x = x;
  a.y = y;
  int err = qmm::launch_gemv(a, stream);
  if (err) return hip_fail(err, "qmm_gemv");
  return QMM_OK;
}

}  // extern "C"

namespace {

// qmm_gemm and its allocation-free variant: the same validation and kernels,
// the split-K partials in the caller's workspace or in the static scratch.
qmm_status gemm_impl(const char* name, bool noalloc, qmm_format f, const void* packed, int64_t t,
                     int64_t n, int64_t d, const qmm_bf16* x, qmm_bf16* y, void* ws, size_t ws_bytes,
                     void* stream) {
  g_last_error[0] = 0;
  qmm::Layout l;
  qmm_status st = check_shape(f, n, d, &l);
  if (st) return st;
  if (t < 1) return fail(QMM_E_ARG, "t must be >= 1");
  if (t > qmm::kMaxT) return fail(QMM_E_SHAPE, "t must be <= 2^24");
  if (!packed || !x || !y) return fail(QMM_E_ARG, "NULL pointer");
  if (!aligned(packed, 256)) return fail(QMM_E_ALIGN, "packed must be 256-byte aligned");
  if (!aligned(x, 16)) return fail(QMM_E_ALIGN, "x must be 16-byte aligned");
  if (!aligned(y, 2)) return fail(QMM_E_ALIGN, "y must be 2-byte aligned");
  int kf;
  if ((st = check_kernel(&kf))) return st;
  if (kf == QMM_KERNEL_FEW_ROW && !qmm::skinny_fits(t, n, d, l))
    return fail(QMM_E_UNSUPPORTED, "the few-row kernel takes 2 <= t <= 64 rows (kernel forced to few_row)");
  if (kf == QMM_KERNEL_MULTI_ROW && !qmm::mrow_fits(f, t, n, d, l))
    return fail(QMM_E_UNSUPPORTED, "the multi-row kernel takes 2 <= t <= 16 rows whose padded rows fit in 160 KiB of LDS, or 17 <= t <= 64 (kernel forced to multi_row)");
  const size_t need = gemm_ws_bytes(kf, f, t, n, d, l);
  if (noalloc) {
    if (need > qmm::kNoAllocScratchBytes)
      return fail(QMM_E_WORKSPACE, "the split-K partials of this shape exceed the 64 MiB static scratch of qmm_gemm_noalloc");
    ws = nullptr;
    ws_bytes = 0;
    if (need) {
      const int err = qmm::noalloc_scratch(stream, &ws);
      if (err) return hip_fail(err, name);
      ws_bytes = qmm::kNoAllocScratchBytes;
    }
  }
  if ((st = check_ws(need, ws, ws_bytes))) return st;
  if (t == 1 && !forces_tile(kf)) return qmm_gemv(f, packed, n, d, x, y, nullptr, 0, stream);
  qmm::GemmArgs a{};
  a.f = f;
  a.packed = static_cast<const uint8_t*>(packed);
  a.t = int(t);
  a.n = int(n);
  a.d = int(d);
  a.x = x;
  a.y = y;
  if (uses_mrow(kf, f, t, n, d, l)) {
    const int err = qmm::launch_mrow(a, stream);
    if (err) return hip_fail(err, name);
    return QMM_OK;
  }
  if (f == QMM_AFFINE4_G64 && !ws)
    return fail(QMM_E_WORKSPACE, "affine weights on the matmul kernels need a workspace of qmm_workspace_bytes() bytes");
  if (kf == QMM_KERNEL_FEW_ROW && !ws)
    return fail(QMM_E_WORKSPACE, "the few-row kernel needs a workspace of qmm_workspace_bytes() bytes");
  if (need && ws && !aligned(ws, 16)) return fail(QMM_E_ALIGN, "ws must be 16-byte aligned");
  // the tile kernel is told only the workspace bytes it may use: without the
  // K-split planes when it must not split
  const size_t tile_bytes = kf == QMM_KERNEL_TILE_UNSPLIT ? need : ws_bytes;
  int err = ws && !forces_tile(kf) && qmm::skinny_fits(t, n, d, l)
                ? qmm::launch_skinny(a, static_cast<float*>(ws), stream)
                : qmm::launch_gemm_ws(a, need ? static_cast<float*>(ws) : nullptr, need ? tile_bytes : 0, stream);
  if (err) return hip_fail(err, name);
  return QMM_OK;
}

}  // namespace

extern "C" {

qmm_status qmm_gemm(qmm_format f, const void* packed, int64_t t, int64_t n, int64_t d,
                    const qmm_bf16* x, qmm_bf16* y, void* ws, size_t ws_bytes, void* stream) {
  return gemm_impl("qmm_gemm", false, f, packed, t, n, d, x, y, ws, ws_bytes, stream);
}

qmm_status qmm_gemm_noalloc(qmm_format f, const void* packed, int64_t t, int64_t n, int64_t d,
                            const qmm_bf16* x, qmm_bf16* y, void* stream) {
  return gemm_impl("qmm_gemm_noalloc", true, f, packed, t, n, d, x, y, nullptr, 0, stream);
}

namespace {

qmm_status grouped(const char* name, bool swiglu, qmm_format f, const void* packed_stack,
                   int64_t expert_stride_bytes, int32_t n_experts, int64_t n, int64_t d,
                   const qmm_bf16* x, int64_t t_x, const int32_t* row_index,
                   const int32_t* seg_expert, const int32_t* seg_offsets, int32_t n_seg,
                   int32_t m_total, int32_t max_seg_rows, qmm_bf16* y, void* ws, size_t ws_bytes,
                   void* stream) {
  g_last_error[0] = 0;
  qmm::Layout l;
  qmm_status st = check_shape(f, n, d, &l);
  if (st) return st;
  if (swiglu && n % 2) return fail(QMM_E_SHAPE, "a gate_up stack needs an even n (gate rows, then up rows)");
  if (n_experts < 1) return fail(QMM_E_ARG, "n_experts must be >= 1");
  if (expert_stride_bytes < l.total_bytes || expert_stride_bytes % 256)
    return fail(QMM_E_ARG, "expert_stride_bytes must be a multiple of 256 and >= qmm_packed_bytes");
  if (n_seg < 0 || m_total < 0 || t_x < 1) return fail(QMM_E_ARG, "n_seg, m_total >= 0 and t_x >= 1 required");
  if (n_seg > 65535) return fail(QMM_E_SHAPE, "n_seg must be <= 65535");
  if (!packed_stack || !x || !y) return fail(QMM_E_ARG, "NULL pointer");
  if (n_seg > 0 && (!seg_expert || !seg_offsets)) return fail(QMM_E_ARG, "NULL routing table");
  if (n_seg > 0 && max_seg_rows < 1) return fail(QMM_E_ARG, "max_seg_rows must be >= 1");
  if (!aligned(packed_stack, 256)) return fail(QMM_E_ALIGN, "packed_stack must be 256-byte aligned");
  if (!aligned(x, 16)) return fail(QMM_E_ALIGN, "x must be 16-byte aligned");
  if (!aligned(y, 2)) return fail(QMM_E_ALIGN, "y must be 2-byte aligned");
  if (!aligned(row_index, 4) || !aligned(seg_expert, 4) || !aligned(seg_offsets, 4))
    return fail(QMM_E_ALIGN, "routing tables must be 4-byte aligned");
  if ((st = check_ws(0, ws, ws_bytes))) return st;
  int kf;
  if ((st = check_kernel(&kf))) return st;
  if (n_seg == 0 || m_total == 0) return QMM_OK;
  int err;
  // one row per segment takes the decode GEMV, unless the activation is
  // fused or the rows are taken in order (the matmul kernel does both), or
  // the matmul kernel is forced
  if (max_seg_rows == 1 && !swiglu && row_index && gemv_fits(n, d, l) && kf != QMM_KERNEL_GROUPED_MATMUL) {
    qmm::GemvArgs a{};
    a.f = f;
    a.packed = static_cast<const uint8_t*>(packed_stack);
    a.expert_stride = expert_stride_bytes;
    a.n_experts = n_experts;
    a.n = int(n);
    a.d = int(d);
    a.x = x;
    a.t_x = t_x;
    a.row_index = row_index;
    a.seg_expert = seg_expert;
    a.seg_offsets = seg_offsets;
    a.n_seg = n_seg;
    a.m_total = m_total;
    a.y = y;
    err = qmm::launch_gemv(a, stream);
  } else if (kf != QMM_KERNEL_GROUPED_MATMUL && max_seg_rows <= qmm::kMrowGroupedMaxT &&
             qmm::mrow_grouped_fits(f, swiglu ? std::max(max_seg_rows, 2) : max_seg_rows, n, d, t_x, l)) {
    // a few rows per segment: the multi-row kernel reads each expert's
    // weights once for all of them (with the activation: also one row)
    qmm::MrowGroupedArgs a{};
    a.f = f;
    a.stack = static_cast<const uint8_t*>(packed_stack);
    a.grp.expert_stride = expert_stride_bytes;
    a.grp.row_index = row_index;
    a.grp.seg_expert = seg_expert;
    a.grp.seg_offsets = seg_offsets;
    a.grp.n_experts = n_experts;
    a.grp.m_total = m_total;
    a.grp.t_x = int(t_x);
    a.n_seg = n_seg;
    a.t = swiglu ? std::max(max_seg_rows, 2) : max_seg_rows;
    a.n = int(n);
    a.d = int(d);
    a.x = x;
    a.y = y;
    a.glu = swiglu;
    err = qmm::launch_mrow_grouped(a, stream);
  } else {
    // longer segments: the matmul kernel; the short ones among them (up to
    // the multi-row kernel's bound, found on the device) go to the multi-row
    // kernel first
    const bool split = kf != QMM_KERNEL_GROUPED_MATMUL && max_seg_rows > qmm::kMrowGroupedMaxT &&
                       qmm::mrow_grouped_fits(f, qmm::kMrowGroupedMaxT, n, d, t_x, l);
    if (split) {
      // armed profiling events: the start with the first launch, the stop
      // with the second
      const qmm::ProfileEvents pe = qmm::take_profile_events();
      g_profile = {pe.start, nullptr};
      qmm::MrowGroupedArgs a{};
      a.f = f;
      a.stack = static_cast<const uint8_t*>(packed_stack);
      a.grp.expert_stride = expert_stride_bytes;
      a.grp.row_index = row_index;
      a.grp.seg_expert = seg_expert;
      a.grp.seg_offsets = seg_offsets;
      a.grp.n_experts = n_experts;
      a.grp.m_total = m_total;
      a.grp.t_x = int(t_x);
      a.grp.max_rows = qmm::kMrowGroupedMaxT;
      a.n_seg = n_seg;
      a.t = qmm::kMrowGroupedMaxT;
      a.n = int(n);
      a.d = int(d);
      a.x = x;
      a.y = y;
      a.glu = swiglu;
      err = qmm::launch_mrow_grouped(a, stream);
      g_profile = {nullptr, pe.stop};
      if (err) {
        g_profile = {nullptr, nullptr};
        return hip_fail(err, name);
      }
    }
    qmm::GemmArgs a{};
    a.f = f;
    a.packed = static_cast<const uint8_t*>(packed_stack);
    a.expert_stride = expert_stride_bytes;
    a.n_experts = n_experts;
    a.n = int(n);
    a.d = int(d);
    a.x = x;
    a.t_x = t_x;
    a.row_index = row_index;
    a.seg_expert = seg_expert;
    a.seg_offsets = seg_offsets;
    a.n_seg = n_seg;
    a.m_total = m_total;
    a.max_seg_rows = max_seg_rows;
    a.y = y;
    a.swiglu = swiglu;
    err = qmm::launch_grouped_gemm_long(a, split ? qmm::kMrowGroupedMaxT : 0, stream);
  }
  if (err) return hip_fail(err, name);
  return QMM_OK;
}

}  // namespace

qmm_status qmm_grouped_gemm(qmm_format f, const void* packed_stack, int64_t expert_stride_bytes,
                            int32_t n_experts, int64_t n, int64_t d, const qmm_bf16* x,
                            int64_t t_x, const int32_t* row_index, const int32_t* seg_expert,
                            const int32_t* seg_offsets, int32_t n_seg, int32_t m_total,
                            int32_t max_seg_rows, qmm_bf16* y, void* ws, size_t ws_bytes,
                            void* stream) {
  return grouped("qmm_grouped_gemm", false, f, packed_stack, expert_stride_bytes, n_experts, n, d, x,
                 t_x, row_index, seg_expert, seg_offsets, n_seg, m_total, max_seg_rows, y, ws,
                 ws_bytes, stream);
}

qmm_status qmm_grouped_gemm_swiglu(qmm_format f, const void* packed_stack,
                                   int64_t expert_stride_bytes, int32_t n_experts, int64_t n,
                                   int64_t d, const qmm_bf16* x, int64_t t_x,
                                   const int32_t* row_index, const int32_t* seg_expert,
                                   const int32_t* seg_offsets, int32_t n_seg, int32_t m_total,
                                   int32_t max_seg_rows, qmm_bf16* h, void* ws, size_t ws_bytes,
                                   void* stream) {
  return grouped("qmm_grouped_gemm_swiglu", true, f, packed_stack, expert_stride_bytes, n_experts, n,
                 d, x, t_x, row_index, seg_expert, seg_offsets, n_seg, m_total, max_seg_rows, h, ws,
                 ws_bytes, stream);
}

qmm_status qmm_gemv_int8(qmm_format f, const void* packed, int64_t n, int64_t d, const qmm_bf16* x,
                         qmm_bf16* y, void* stream) {
  g_last_error[0] = 0;
  if (f != QMM_AFFINE4_G64) return fail(f == QMM_MXFP4_G32 ? QMM_E_UNSUPPORTED : QMM_E_ARG,
                                        "the deferred-dequantisation GEMV takes affine weights");
  qmm::Layout l;
  qmm_status st = check_shape(f, n, d, &l);
  if (st) return st;
  if (d > qmm::kI8MaxD) return fail(QMM_E_SHAPE, "d must be <= 57344 (the row's int8 codes live in LDS)");
  if (!gemv_fits(n, d, l)) return fail(QMM_E_SHAPE, "n*d/2 must be below 2^31");
  if (!packed || !x || !y) return fail(QMM_E_ARG, "NULL pointer");
  if (!aligned(packed, 256)) return fail(QMM_E_ALIGN, "packed must be 256-byte aligned");
  if (!aligned(x, 16)) return fail(QMM_E_ALIGN, "x must be 16-byte aligned");
  if (!aligned(y, 2)) return fail(QMM_E_ALIGN, "y must be 2-byte aligned");
  qmm::GemvArgs a{};
  a.f = f;
  a.packed = static_cast<const uint8_t*>(packed);
  a.n = int(n);
  a.d = int(d);
  a.x = x;
  a.y = y;
  const int err = qmm::launch_gemv_i8(a, stream);
  if (err) return hip_fail(err, "qmm_gemv_int8");
  return QMM_OK;
}

qmm_status qmm_moe_combine(const qmm_bf16* o, int32_t m_total, int64_t d, int64_t t, int32_t k,
                           const int32_t* topk, const float* weights, int32_t n_experts,
                           const int32_t* seg_offsets, const int32_t* row_index, qmm_bf16* out,
                           void* stream) {
  g_last_error[0] = 0;
  if (!o || !topk || !weights || !seg_offsets || !row_index || !out) return fail(QMM_E_ARG, "NULL pointer");
  if (t < 1 || k < 1 || n_experts < 1 || m_total < 0) return fail(QMM_E_ARG, "t, k, n_experts >= 1 and m_total >= 0 required");
  if (k > qmm::kCombineMaxK) return fail(QMM_E_SHAPE, "k must be <= 64");
  if (d < 8 || d % 8 || d > qmm::kMaxD) return fail(QMM_E_SHAPE, "d must be a multiple of 8 in [8, 65536]");
  if (t * k >= (int64_t(1) << 31) || t > (int64_t(1) << 31) - 1) return fail(QMM_E_SHAPE, "t*k must be below 2^31");
  if (!aligned(o, 16) || !aligned(out, 16)) return fail(QMM_E_ALIGN, "o and out must be 16-byte aligned");
  if (!aligned(topk, 4) || !aligned(weights, 4) || !aligned(seg_offsets, 4) || !aligned(row_index, 4))
    return fail(QMM_E_ALIGN, "tables and weights must be 4-byte aligned");
  qmm::CombineArgs a{o, m_total, int(d), int(t), k, topk, weights, n_experts, seg_offsets, row_index, out};
  const int err = qmm::launch_combine(a, stream);
  if (err) return hip_fail(err, "qmm_moe_combine");
  return QMM_OK;
}

}  // extern "C"
