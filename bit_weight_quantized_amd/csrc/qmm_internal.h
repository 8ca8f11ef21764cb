// Internal definitions shared by the qmm library sources (host and device).
//
// Packed device layout, version 4 (written by qmm_pack, read by every kernel):
//
//   [0, 256)            header (PackedHeader)
//   [256, meta_off)     codes, K-slabbed
//   [meta_off, total)   per-group metadata, quad-major
//
// K-slabbed codes: the reduction axis is cut into slabs of 512 codes (the last
// slab may be narrower, any multiple of 32).  Slab s stores its width w_s of
// every row, rows consecutive, and the slabs follow one another:
//   codes of (slab s, row r) at  s·n·256 + r·w_s/2
// A decode GEMV sweeps the matrix slab by slab with all rows in flight, so at
// any moment the whole GPU reads one contiguous window of memory, and each wave
// load instruction covers 4 rows × 256 bytes = 1 KiB contiguous.
//
// Quad-major metadata: rows are taken in quads (4 consecutive rows; n is
// padded to a multiple of 4 with zero metadata).  A quad's metadata is one
// contiguous block of 4·M bytes, M the metadata bytes of one row, ordered
// slab by slab and, inside a slab, row by row:
//   metadata of (slab s, row r) at  (r / 4)·4M + 4·s·m_full + (r % 4)·m_s
// where m_s is the metadata bytes of one row in slab s: (w_s/64)·4 for affine,
// w_s/32 rounded up to a multiple of 4 for MXFP4 (padding bytes are zero), so
// every row's metadata starts 4-byte aligned and can be fetched as dwords, and
// m_full = m_s of a full slab (32 affine, 16 MXFP4).  A GEMV wave fetches its
// quad's metadata for a run of slabs as one contiguous piece; a GEMM column
// block reads 4 rows of a slab from one 128- (64-) byte segment.
//
// affine codes: one uint32 per 8 codes, nibbles regrouped so that the low
//   half-word holds the even codes and the high half-word the odd codes:
//   bits 4i..4i+3 = q[8w + 2i], bits 16+4i..16+4i+3 = q[8w + 2i + 1], i = 0..3.
//   (w >> 4i) & 0x000F000F then isolates the consecutive pair (q[2i], q[2i+1])
//   in the two bf16 lanes of a register, ready for a 2-wide bf16 dot with the
//   matching pair of activations.
// affine metadata: uint32 per group, bf16 scale in the low half, bf16 bias in
//   the high half (4 bytes per 64 codes, so 36 bytes per group in total).
// MXFP4 codes: the canonical byte order (even code in the low nibble), which
//   is the order the gfx950 FP4 -> bf16 pair conversion consumes.
// MXFP4 metadata: the E8M0 bytes, one per 32 codes.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "../../include/qmm.h"

namespace qmm {

constexpr uint32_t kMagic = 0x344D4D51u;  // "QMM4"
constexpr uint32_t kLayoutVersion = 4;
constexpr uint32_t kFlagInvalid = 1u;     // set by qmm_pack when an E8M0 byte is 255
constexpr int64_t kHeaderBytes = 256;
constexpr int64_t kMaxN = int64_t(1) << 28;  // keeps every grid below 2^32 work-items
constexpr int64_t kMaxD = 65536;
constexpr int64_t kMaxT = int64_t(1) << 24;

struct PackedHeader {
  uint32_t magic;
  uint32_t version;
  uint32_t format;
  uint32_t flags;
  int64_t n;
  int64_t d;
  int64_t codes_offset;
  int64_t meta_offset;
  int64_t total_bytes;
};
static_assert(sizeof(PackedHeader) <= kHeaderBytes, "header too large");

inline int group_of(int f) { return f == QMM_AFFINE4_G64 ? 64 : (f == QMM_MXFP4_G32 ? 32 : 0); }

inline int64_t round_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

struct Layout {
  int64_t codes_offset, meta_offset, meta_bytes, total_bytes;
};

// metadata bytes of one row: 4 per 64 codes (affine), or one byte per 32
// codes with each slab's bytes padded to a multiple of 4 (MXFP4; only the
// last slab can be narrower than 512 codes)
inline int64_t row_meta_bytes(int f, int64_t d) {
  if (f == QMM_AFFINE4_G64) return d / 16;
  const int64_t wl = d - (d - 1) / 512 * 512;  // width of the last slab
  return (d - wl) / 32 + round_up(wl / 32, 4);
}

inline bool layout_of(int f, int64_t n, int64_t d, Layout* out) {
  const int g = group_of(f);
  if (g == 0 || n < 1 || n > kMaxN || d < g || d > kMaxD || d % g) return false;
  Layout l;
  l.codes_offset = kHeaderBytes;
  l.meta_offset = round_up(l.codes_offset + n * (d / 2), 256);
  l.meta_bytes = round_up(n, 4) * row_meta_bytes(f, d);
  l.total_bytes = round_up(l.meta_offset + l.meta_bytes, 256);
  *out = l;
  return true;
}

// Geometry of the K-slabbed layout (bytes relative to the codes / metadata
// section starts).
constexpr int kSlabCodes = 512;

struct Slabs {
  int64_t n;
  int d;
  int fmt;
  __host__ __device__ int count() const { return (d + kSlabCodes - 1) / kSlabCodes; }
  __host__ __device__ int width(int s) const {
    const int w = d - kSlabCodes * s;
    return w < kSlabCodes ? w : kSlabCodes;
  }
  __host__ __device__ int64_t codes(int s, int64_t row) const {
    return int64_t(s) * n * (kSlabCodes / 2) + row * (width(s) / 2);
  }
  // metadata bytes of one row in slab s, and in a full slab
  __host__ __device__ int meta_row(int s) const {
    return fmt == QMM_AFFINE4_G64 ? width(s) / 16 : (width(s) / 32 + 3) & ~3;
  }
  __host__ __device__ int meta_full() const { return fmt == QMM_AFFINE4_G64 ? 32 : 16; }
  // metadata bytes of one quad (4 rows, all slabs)
  __host__ __device__ int64_t meta_quad() const {
    return 4 * (int64_t(count() - 1) * meta_full() + meta_row(count() - 1));
  }
  __host__ __device__ int64_t meta(int s, int64_t row) const {
    return (row >> 2) * meta_quad() + 4 * int64_t(s) * meta_full() + (row & 3) * meta_row(s);
  }
  // byte offsets of code k / of the metadata of the group holding code k
  __host__ __device__ int64_t code_byte(int64_t row, int k) const {
    return codes(k / kSlabCodes, row) + (k % kSlabCodes) / 2;
  }
  __host__ __device__ int64_t meta_byte(int64_t row, int k) const {
    return meta(k / kSlabCodes, row) +
           (fmt == QMM_AFFINE4_G64 ? 4 * ((k % kSlabCodes) / 64) : (k % kSlabCodes) / 32);
  }
};

}  // namespace qmm

// ---------------------------------------------------------------------------
// Launchers implemented in the .hip files (host side, return hipError_t as int)
// ---------------------------------------------------------------------------
namespace qmm {

// Events armed by qmm_profile_next() for the next hot-path launch on this
// thread; take_profile_events() returns and disarms them.
struct ProfileEvents {
  void* start;
  void* stop;
};
ProfileEvents take_profile_events();

struct DevInfo {
  int cus;
};
int device_info(DevInfo* out);  // 0 on success, else a hipError_t

int launch_pack(int f, int64_t n, int64_t d, const void* codes, const void* scales,
                const void* biases, void* packed, void* stream);
int launch_unpack(int f, int64_t n, int64_t d, const void* packed, void* codes, void* scales,
                  void* biases, void* stream);
int read_header(const void* packed, PackedHeader* out, void* stream);

struct GemvArgs {
  int f;
  const uint8_t* packed;         // blob (dense) or stack (grouped)
  int64_t expert_stride;         // grouped only
  int n_experts;                 // grouped only
  int n, d;
  const uint16_t* x;
  int64_t t_x;                   // grouped: rows of x
  const int32_t* row_index;      // grouped only
  const int32_t* seg_expert;     // grouped only
  const int32_t* seg_offsets;    // grouped only
  int n_seg;                     // grouped only (0 = dense)
  int m_total;                   // grouped only
  uint16_t* y;
};
int launch_gemv(const GemvArgs& a, void* stream);

struct GemmArgs {
  int f;
  const uint8_t* packed;
  int64_t expert_stride;
  int n_experts;
  int t, n, d;
  const uint16_t* x;
  int64_t t_x;
  const int32_t* row_index;
  const int32_t* seg_expert;
  const int32_t* seg_offsets;
  int n_seg;
  int m_total;
  int max_seg_rows;
  uint16_t* y;
  bool swiglu = false;   // grouped: y = silu(gate)·up of a gate_up stack, [m_total][n/2]
};
int launch_gemm(const GemmArgs& a, void* stream);
int launch_grouped_gemm(const GemmArgs& a, void* stream);

constexpr int kCombineMaxK = 64;
struct CombineArgs {
  const uint16_t* o;   // [m_total, d] bf16, grouped order
  int m_total, d, t, k;
  const int32_t* topk;       // [t, k]
  const float* weights;      // [t, ne] routing weights
  int ne;
  const int32_t* seg_offsets;   // [ne + 1], dense per expert
  const int32_t* row_index;     // [m_total], tokens ascending within a segment
  uint16_t* out;             // [t, d] bf16
};
int launch_combine(const CombineArgs& a, void* stream);

struct RouteArgs {
  const uint16_t* x;   // [t, d] bf16
  int t, d;
  const uint16_t* r;   // [ne, d] bf16
  int ne;
  const float* bias;   // [ne] or NULL
  int k;
  float* scores;       // [t, ne]
  int32_t* topk;       // [t, k]
  int32_t* seg_expert;   // [ne]
  int32_t* seg_offsets;  // [ne + 1]
  int32_t* row_index;    // [t * k]
};
constexpr int kRouteMaxExperts = 1024;
constexpr int kRouteMaxK = 64;
int launch_route(const RouteArgs& a, void* stream);

// read-only streaming kernel (measurement support): kStreamBlocks workgroups
constexpr int kStreamBlocks = 2048;
int launch_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream);

}  // namespace qmm
