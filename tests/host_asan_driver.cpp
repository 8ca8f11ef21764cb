// Host-only driver for the C-ABI validation of libqmm (csrc/qmm_api.cpp),
// built with g++ -fsanitize=address by tests/test_host_asan.py.  The HIP
// launchers are replaced by stubs that record which launcher a call reached
// and with what, so every validation branch, the status and error-text paths
// and the kernel selection run on the CPU under AddressSanitizer; no GPU and
// no HIP runtime are involved.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <string>

#include "../bit_weight_quantized_amd/csrc/qmm_deferred.h"
#include "../bit_weight_quantized_amd/csrc/qmm_internal.h"
#include "../bit_weight_quantized_amd/csrc/qmm_mrow.h"
#include "../bit_weight_quantized_amd/csrc/qmm_skinny.h"

// ---- stubs -----------------------------------------------------------------
static std::string g_called;      // the launcher the last call reached
static int g_fail = 0;            // error the next launcher returns (then reset)
static uint32_t g_header_flags = 0;
static int64_t g_header_n = 16, g_header_d = 64;
static const void* g_ws = nullptr;
static size_t g_ws_bytes = 0;
alignas(256) static unsigned char g_scratch[512];

static int reach(const char* name) {
  g_called = name;
  const int f = g_fail;
  g_fail = 0;
  return f;
}

extern "C" const char* hipGetErrorString(hipError_t) { return "stub HIP error with a long description text"; }

namespace qmm {
int launch_gemv(const GemvArgs&, void*) { return reach("gemv"); }
int launch_pack(int, int64_t, int64_t, const void*, const void*, const void*, void*, void*) { return reach("pack"); }
int launch_unpack(int, int64_t, int64_t, const void*, void*, void*, void*, void*) { return reach("unpack"); }
int read_header(const void*, PackedHeader* h, void*) {
  memset(h, 0, sizeof(*h));
  h->magic = kMagic;
  h->version = kLayoutVersion;
  h->format = QMM_AFFINE4_G64;
  h->flags = g_header_flags;
  h->n = g_header_n;
  h->d = g_header_d;
  return 0;
}
int launch_route(const RouteArgs&, void*) { return reach("route"); }
int launch_skinny(const GemmArgs&, float* ws, void*) { g_ws = ws; return reach("skinny"); }
int launch_mrow(const GemmArgs&, void*) { return reach("mrow"); }
int launch_mrow_grouped(const MrowGroupedArgs&, void*) { return reach("mrow_grouped"); }
int launch_combine(const CombineArgs&, void*) { return reach("combine"); }
int launch_gemm_ws(const GemmArgs&, float* ws, size_t bytes, void*) {
  g_ws = ws;
  g_ws_bytes = bytes;
  return reach("gemm_ws");
}
int launch_gemv_i8(const GemvArgs&, void*) { return reach("gemv_i8"); }
int noalloc_scratch(void*, void** out) {
  *out = g_scratch;
  return reach("scratch") ? 1 : 0;
}
int launch_stream_read(const void*, size_t, uint32_t*, void*) { return reach("stream_read"); }
int launch_grouped_gemm(const GemmArgs&, void*) { return reach("grouped_gemm"); }
// the matmul kernel over the segments longer than skip_rows: after the
// multi-row kernel took the short ones (a split call), or alone
int launch_grouped_gemm_long(const GemmArgs&, int skip_rows, void*) {
  if (skip_rows == 0) return reach("grouped_gemm");
  return reach(skip_rows == kMrowGroupedMaxT && g_called == "mrow_grouped" ? "split" : "bad_split");
}
}  // namespace qmm

// ---- checks ----------------------------------------------------------------
static int g_bad = 0;
#define EXPECT(cond)                                                      \
  do {                                                                    \
    if (!(cond)) {                                                        \
      fprintf(stderr, "FAILED line %d: %s (last error: %s, called: %s)\n", \
              __LINE__, #cond, qmm_last_error(), g_called.c_str());       \
      ++g_bad;                                                            \
    }                                                                     \
  } while (0)

static void* P(uintptr_t off = 0) { return reinterpret_cast<void*>((uintptr_t(1) << 20) + off); }
static qmm_bf16* B(uintptr_t off = 0) { return static_cast<qmm_bf16*>(P(off)); }
static int32_t* I(uintptr_t off = 0) { return static_cast<int32_t*>(P(off)); }

int main() {
  const qmm_format A = QMM_AFFINE4_G64, M = QMM_MXFP4_G32;
  const size_t blob = qmm_packed_bytes(A, 16, 64);
  EXPECT(blob % 256 == 0 && blob >= 256 + 16 * 64 * 36 / 64);
  EXPECT(qmm_packed_bytes(A, 16, 96) == 0 && qmm_packed_bytes(static_cast<qmm_format>(3), 16, 64) == 0);

  // every status has its own text; unknown codes are named as such
  for (int s = 0; s <= 8; ++s) EXPECT(strcmp(qmm_status_string(static_cast<qmm_status>(s)), "unknown status") != 0);
  EXPECT(strcmp(qmm_status_string(static_cast<qmm_status>(99)), "unknown status") == 0);

  // GEMV: shape, pointer and alignment errors launch nothing
  g_called = "none";
  EXPECT(qmm_gemv(static_cast<qmm_format>(7), P(), 16, 64, B(), B(), nullptr, 0, nullptr) == QMM_E_ARG);
  EXPECT(qmm_gemv(A, P(), 16, 96, B(), B(), nullptr, 0, nullptr) == QMM_E_SHAPE);
  EXPECT(qmm_gemv(M, P(), 16, 48, B(), B(), nullptr, 0, nullptr) == QMM_E_SHAPE);
  EXPECT(qmm_gemv(A, nullptr, 16, 64, B(), B(), nullptr, 0, nullptr) == QMM_E_ARG);
  EXPECT(qmm_gemv(A, P(16), 16, 64, B(), B(), nullptr, 0, nullptr) == QMM_E_ALIGN);
  EXPECT(qmm_gemv(A, P(), 16, 64, B(8), B(), nullptr, 0, nullptr) == QMM_E_ALIGN);
  EXPECT(qmm_gemv(A, P(), int64_t(1) << 27, 65536, B(), B(), nullptr, 0, nullptr) == QMM_E_SHAPE);
  EXPECT(g_called == "none");
  EXPECT(qmm_gemv(A, P(), 16, 64, B(), B(), nullptr, 0, nullptr) == QMM_OK && g_called == "gemv");
  EXPECT(qmm_last_error()[0] == 0);

  // GEMM: kernel selection by t and workspace
  EXPECT(qmm_gemm(A, P(), 1, 16, 64, B(), B(), nullptr, 0, nullptr) == QMM_OK && g_called == "gemv");
  // a few rows on a wide matrix: the multi-row kernel, no workspace (one
  // passed is ignored)
  EXPECT(qmm_workspace_bytes(A, 8, 13824, 5120) == 0);
  EXPECT(qmm_gemm(A, P(), 8, 13824, 5120, B(), B(), nullptr, 0, nullptr) == QMM_OK && g_called == "mrow");
  EXPECT(qmm_gemm(A, P(), 8, 13824, 5120, B(), B(), P(8), 16, nullptr) == QMM_OK && g_called == "mrow");
  EXPECT(qmm_gemm(M, P(), 4, 1024, 5120, B(), B(), nullptr, 0, nullptr) == QMM_OK && g_called == "mrow");
  g_fail = 1;   // a launch error is reported as a HIP status
  EXPECT(qmm_gemm(A, P(), 8, 13824, 5120, B(), B(), nullptr, 0, nullptr) == QMM_E_HIP);
  // narrower: the few-row split-K kernel through the workspace
  const size_t need8 = qmm_workspace_bytes(A, 8, 4096, 5120);
  EXPECT(need8 == size_t(10) * 8 * 4096 * 4);
  EXPECT(qmm_gemm(A, P(), 8, 4096, 5120, B(), B(), P(), need8, nullptr) == QMM_OK && g_called == "skinny");
  EXPECT(qmm_gemm(A, P(), 8, 4096, 5120, B(), B(), P(), need8 - 1, nullptr) == QMM_E_WORKSPACE);
  EXPECT(qmm_gemm(A, P(), 8, 4096, 5120, B(), B(), P(8), need8, nullptr) == QMM_E_ALIGN);
  EXPECT(qmm_gemm(A, P(), 8, 4096, 5120, B(), B(), nullptr, 0, nullptr) == QMM_E_WORKSPACE);
  g_called = "none";
  EXPECT(qmm_gemm(A, P(), 0, 16, 64, B(), B(), nullptr, 0, nullptr) == QMM_E_ARG && g_called == "none");
  EXPECT(qmm_gemm(A, P(), (int64_t(1) << 24) + 1, 16, 64, B(), B(), nullptr, 0, nullptr) == QMM_E_SHAPE);
  EXPECT(qmm_gemm(M, P(), 2048, 13824, 5120, B(), B(), nullptr, 0, nullptr) == QMM_OK && g_called == "gemm_ws");
  EXPECT(g_ws == nullptr && g_ws_bytes == 0);
  // affine weights through the tile kernel need the workspace (fp16 activations)
  const size_t need2k = qmm_workspace_bytes(A, 2048, 13824, 5120);
  EXPECT(need2k == size_t(2048) * 5120 * 2 + 2048 * 4 + 13824 * 4);
  EXPECT(qmm_gemm(A, P(), 2048, 13824, 5120, B(), B(), nullptr, 0, nullptr) == QMM_E_WORKSPACE);
  EXPECT(qmm_gemm(A, P(), 2048, 13824, 5120, B(), B(), P(), need2k, nullptr) == QMM_OK && g_called == "gemm_ws");
  EXPECT(g_ws == P() && g_ws_bytes == need2k);
  EXPECT(qmm_gemm(A, P(), 3, 16, 5120, B(), B(), P(), qmm_workspace_bytes(A, 3, 16, 5120), nullptr) == QMM_OK &&
         g_called == "skinny");
  // short reductions (d <= 3072) take the multi-row kernel at any width
  EXPECT(qmm_gemm(A, P(), 3, 16, 3072, B(), B(), nullptr, 0, nullptr) == QMM_OK && g_called == "mrow");

  // the allocation-free GEMM: the static scratch replaces the workspace; too
  // large a shape is refused before the scratch is looked up
  g_called = "none";
  EXPECT(qmm_gemm_noalloc(A, P(), 64, 6000, 32768, B(), B(), nullptr) == QMM_E_WORKSPACE && g_called == "none");
  EXPECT(strstr(qmm_last_error(), "64 MiB") != nullptr);
  EXPECT(qmm_gemm_noalloc(A, P(), 8, 13824, 5120, B(), B(), nullptr) == QMM_OK && g_called == "mrow");
  EXPECT(qmm_gemm_noalloc(A, P(), 8, 4096, 5120, B(), B(), nullptr) == QMM_OK && g_called == "skinny");
  // 17 <= t <= 64: streamed multi-row rows wherever d <= 2048, from 6912
  // columns while d <= 5120 and from 10240 beyond; the few-row kernel below
  EXPECT(qmm_gemm_noalloc(A, P(), 40, 13824, 5120, B(), B(), nullptr) == QMM_OK && g_called == "mrow");
  EXPECT(qmm_gemm_noalloc(M, P(), 40, 300, 2048, B(), B(), nullptr) == QMM_OK && g_called == "mrow");
  EXPECT(qmm_gemm_noalloc(A, P(), 40, 6912, 5120, B(), B(), nullptr) == QMM_OK && g_called == "mrow");
  EXPECT(qmm_gemm_noalloc(M, P(), 40, 10240, 8192, B(), B(), nullptr) == QMM_OK && g_called == "mrow");
  EXPECT(qmm_gemm_noalloc(M, P(), 40, 2047, 2560, B(), B(), nullptr) == QMM_OK && g_called == "skinny");
  EXPECT(qmm_gemm_noalloc(A, P(), 40, 6911, 5120, B(), B(), nullptr) == QMM_OK && g_called == "skinny");
  EXPECT(qmm_gemm_noalloc(M, P(), 40, 8192, 8192, B(), B(), nullptr) == QMM_OK && g_called == "skinny");
  EXPECT(g_ws == g_scratch);
  g_fail = 1;   // the scratch lookup fails: a HIP status, with the HIP text
  EXPECT(qmm_gemm_noalloc(A, P(), 8, 4096, 5120, B(), B(), nullptr) == QMM_E_HIP);
  EXPECT(strstr(qmm_last_error(), "qmm_gemm_noalloc") != nullptr);
  // the multi-row kernel forced: narrow matrices too; shapes it does not
  // take are refused before any launch
  EXPECT(qmm_set_kernel(QMM_KERNEL_MULTI_ROW) == QMM_OK);
  EXPECT(qmm_gemm(A, P(), 8, 1024, 5120, B(), B(), nullptr, 0, nullptr) == QMM_OK && g_called == "mrow");
  g_called = "none";
  EXPECT(qmm_gemm(A, P(), 17, 13824, 5120, B(), B(), nullptr, 0, nullptr) == QMM_OK && g_called == "mrow");
  EXPECT(qmm_gemm(M, P(), 64, 13824, 5120, B(), B(), nullptr, 0, nullptr) == QMM_OK && g_called == "mrow");
  g_called = "none";
  EXPECT(qmm_gemm(A, P(), 65, 13824, 5120, B(), B(), nullptr, 0, nullptr) == QMM_E_UNSUPPORTED && g_called == "none");
  EXPECT(qmm_gemm(A, P(), 15, 13824, 5120, B(), B(), nullptr, 0, nullptr) == QMM_E_UNSUPPORTED && g_called == "none");
  EXPECT(strstr(qmm_last_error(), "multi-row") != nullptr);
  EXPECT(qmm_set_kernel(QMM_KERNEL_AUTO) == QMM_OK);

  // a launch failure is reported as QMM_E_HIP with the HIP text appended
  g_fail = 1;
  EXPECT(qmm_gemv(A, P(), 16, 64, B(), B(), nullptr, 0, nullptr) == QMM_E_HIP);
  EXPECT(strstr(qmm_last_error(), "stub HIP error") != nullptr);

  // pack / unpack: the header's invalid flag and mismatches
  EXPECT(qmm_pack(A, 16, 64, P(), P(), nullptr, P(), nullptr) == QMM_E_ARG);
  EXPECT(qmm_pack(M, 16, 64, P(), P(), P(), P(), nullptr) == QMM_E_ARG);
  EXPECT(qmm_pack(A, 16, 64, P(), P(), P(), P(64), nullptr) == QMM_E_ALIGN);
  EXPECT(qmm_pack(A, 16, 64, P(2), P(), P(), P(), nullptr) == QMM_E_ALIGN);
  EXPECT(qmm_pack(A, 16, 64, P(), P(), P(), P(), nullptr) == QMM_OK);
  g_header_flags = qmm::kFlagInvalid;
  EXPECT(qmm_pack(A, 16, 64, P(), P(), P(), P(), nullptr) == QMM_E_VALUE);
  EXPECT(qmm_unpack(A, 16, 64, P(), P(), P(), P(), nullptr) == QMM_E_LAYOUT);
  g_header_flags = 0;
  EXPECT(qmm_unpack(A, 16, 64, P(), P(), P(), P(), nullptr) == QMM_OK && g_called == "unpack");
  EXPECT(qmm_unpack(A, 16, 128, P(), P(), P(), P(), nullptr) == QMM_E_LAYOUT);

  // grouped: argument errors, the empty call, the GEMV and matmul selections
  EXPECT(qmm_grouped_gemm(A, P(), blob, 0, 16, 64, B(), 4, I(), I(), I(), 1, 4, 4, B(), nullptr, 0, nullptr) == QMM_E_ARG);
  EXPECT(qmm_grouped_gemm(A, P(), blob - 256, 2, 16, 64, B(), 4, I(), I(), I(), 1, 4, 4, B(), nullptr, 0, nullptr) == QMM_E_ARG);
  EXPECT(qmm_grouped_gemm(A, P(), blob, 2, 16, 64, B(), 4, I(), nullptr, I(), 1, 4, 4, B(), nullptr, 0, nullptr) == QMM_E_ARG);
  EXPECT(qmm_grouped_gemm(A, P(), blob, 2, 16, 64, B(), 4, I(), I(), I(), 70000, 4, 4, B(), nullptr, 0, nullptr) == QMM_E_SHAPE);
  EXPECT(qmm_grouped_gemm(A, P(), blob, 2, 16, 64, B(), 4, I(2), I(), I(), 1, 4, 4, B(), nullptr, 0, nullptr) == QMM_E_ALIGN);
  g_called = "none";
  EXPECT(qmm_grouped_gemm(A, P(), blob, 2, 16, 64, B(), 4, I(), I(), I(), 0, 0, 1, B(), nullptr, 0, nullptr) == QMM_OK && g_called == "none");
  EXPECT(qmm_grouped_gemm(A, P(), blob, 2, 16, 64, B(), 4, I(), I(), I(), 1, 4, 1, B(), nullptr, 0, nullptr) == QMM_OK && g_called == "gemv");
  // 2..8 rows per segment: the multi-row kernel; more, or forced, the matmul kernel
  EXPECT(qmm_grouped_gemm(A, P(), blob, 2, 16, 64, B(), 4, I(), I(), I(), 1, 4, 4, B(), nullptr, 0, nullptr) == QMM_OK && g_called == "mrow_grouped");
  EXPECT(qmm_grouped_gemm(A, P(), blob, 2, 16, 64, B(), 4, nullptr, I(), I(), 1, 4, 8, B(), nullptr, 0, nullptr) == QMM_OK && g_called == "mrow_grouped");
  // more than 8: segments of up to 8 rows to the multi-row kernel, the rest
  // to the matmul kernel (found on the device)
  g_called = "none";
  EXPECT(qmm_grouped_gemm(A, P(), blob, 2, 16, 64, B(), 4, I(), I(), I(), 1, 4, 9, B(), nullptr, 0, nullptr) == QMM_OK && g_called == "split");
  EXPECT(qmm_set_kernel(QMM_KERNEL_GROUPED_MATMUL) == QMM_OK);
  EXPECT(qmm_grouped_gemm(A, P(), blob, 2, 16, 64, B(), 4, I(), I(), I(), 1, 4, 9, B(), nullptr, 0, nullptr) == QMM_OK && g_called == "grouped_gemm");
  EXPECT(qmm_grouped_gemm(A, P(), blob, 2, 16, 64, B(), 4, I(), I(), I(), 1, 4, 4, B(), nullptr, 0, nullptr) == QMM_OK && g_called == "grouped_gemm");
  EXPECT(qmm_set_kernel(QMM_KERNEL_AUTO) == QMM_OK);
  EXPECT(qmm_grouped_gemm_swiglu(A, P(), blob, 2, 15, 64, B(), 4, I(), I(), I(), 1, 4, 4, B(), nullptr, 0, nullptr) == QMM_E_SHAPE);
  // with the activation: the multi-row kernel up to 8 rows (one included),
  // the split above, the matmul kernel when forced
  EXPECT(qmm_grouped_gemm_swiglu(A, P(), blob, 2, 16, 64, B(), 4, I(), I(), I(), 1, 4, 1, B(), nullptr, 0, nullptr) == QMM_OK && g_called == "mrow_grouped");
  EXPECT(qmm_grouped_gemm_swiglu(A, P(), blob, 2, 16, 64, B(), 4, I(), I(), I(), 1, 4, 8, B(), nullptr, 0, nullptr) == QMM_OK && g_called == "mrow_grouped");
  g_called = "none";
  EXPECT(qmm_grouped_gemm_swiglu(A, P(), blob, 2, 16, 64, B(), 4, I(), I(), I(), 1, 4, 9, B(), nullptr, 0, nullptr) == QMM_OK && g_called == "split");
  EXPECT(qmm_set_kernel(QMM_KERNEL_GROUPED_MATMUL) == QMM_OK);
  EXPECT(qmm_grouped_gemm_swiglu(A, P(), blob, 2, 16, 64, B(), 4, I(), I(), I(), 1, 4, 4, B(), nullptr, 0, nullptr) == QMM_OK && g_called == "grouped_gemm");
  EXPECT(qmm_set_kernel(QMM_KERNEL_AUTO) == QMM_OK);

  // router, combine, int8 GEMV, stream read
  EXPECT(qmm_route(nullptr, 4, 64, B(), 8, nullptr, 2, static_cast<float*>(P()), I(), I(), I(), I(), nullptr) == QMM_E_ARG);
  EXPECT(qmm_route(B(), 4, 64, B(), 1025, nullptr, 2, static_cast<float*>(P()), I(), I(), I(), I(), nullptr) == QMM_E_SHAPE);
  EXPECT(qmm_route(B(), 4, 60, B(), 8, nullptr, 2, static_cast<float*>(P()), I(), I(), I(), I(), nullptr) == QMM_E_SHAPE);
  EXPECT(qmm_route(B(), 4, 64, B(), 8, static_cast<float*>(P(2)), 2, static_cast<float*>(P()), I(), I(), I(), I(), nullptr) == QMM_E_ALIGN);
  EXPECT(qmm_route(B(), 4, 64, B(), 8, nullptr, 2, static_cast<float*>(P()), I(), I(), I(), I(), nullptr) == QMM_OK && g_called == "route");
  EXPECT(qmm_moe_combine(B(), 8, 64, 4, 65, I(), static_cast<float*>(P()), 8, I(), I(), B(), nullptr) == QMM_E_SHAPE);
  EXPECT(qmm_moe_combine(B(8), 8, 64, 4, 2, I(), static_cast<float*>(P()), 8, I(), I(), B(), nullptr) == QMM_E_ALIGN);
  EXPECT(qmm_moe_combine(B(), 8, 64, 4, 2, I(), static_cast<float*>(P()), 8, I(), I(), B(), nullptr) == QMM_OK && g_called == "combine");
  EXPECT(qmm_gemv_int8(M, P(), 16, 64, B(), B(), nullptr) == QMM_E_UNSUPPORTED);
  EXPECT(qmm_gemv_int8(A, P(), 16, 57408, B(), B(), nullptr) == QMM_E_SHAPE);
  EXPECT(qmm_gemv_int8(A, P(), 16, 64, B(), B(), nullptr) == QMM_OK && g_called == "gemv_i8");
  uint32_t* sink = static_cast<uint32_t*>(P());
  EXPECT(qmm_stream_read(P(8), 1024, sink, nullptr) == QMM_E_ALIGN);
  EXPECT(qmm_stream_read(P(), 1000, sink, nullptr) == QMM_E_SHAPE);
  EXPECT(qmm_stream_read(P(), 1024, sink, nullptr) == QMM_OK && g_called == "stream_read");

  // profiling events are consumed by the next call and never dereferenced here
  EXPECT(qmm_profile_next(P(), P(64)) == QMM_OK);
  EXPECT(qmm::take_profile_events().start == P() && qmm::take_profile_events().start == nullptr);

  if (g_bad) {
    fprintf(stderr, "%d check(s) failed\n", g_bad);
    return 1;
  }
  printf("host validation ok\n");
  return 0;
}
