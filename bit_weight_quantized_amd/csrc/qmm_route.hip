// MoE router on the GPU: sigmoid scores with a selection-only bias, top-k per
// token, and the tokens grouped by expert for the grouped matmul -- the
// router with a score-correction bias of "Colibri Kimi K3 Metal 后端实现全解析"
// (introduction) and the sigmoid top-16 over 896 routed experts of "Kimi K3
// 迁移到 Google TPU 的可行性评估（v2）" (§2 模型解剖).
//
// Three launches on the caller's stream, no workspace:
//   1. scores[t, e] = sigmoid(Σ_j x[t,j]·R[e,j]) in fp32 (the routing weight): one
//      workgroup per 32 tokens × 32 experts, its eight waves splitting d and
//      staging their pieces through LDS, v_mfma_f32_16x16x32_bf16 with fp32
//      accumulation, tiles ordered so each XCD reads a slice of x and R;
//   2. top-k per token by the selection score fp32(score + bias[e]): one wave
//      per token holds them in registers (up to 16 per lane) as
//      order-preserving integer keys and
//      takes k rounds of a wave-wide maximum (DPP within rows of 16 lanes,
//      then across rows in scalar registers), equal keys going to the lower
//      expert id;
//   3. grouping, one workgroup: per-expert counts with LDS atomics (order free),
//      an exclusive scan into seg_offsets, then tokens in blocks of 512: each
//      assignment sets its bit in an LDS bitmap [expert][512 tokens], the
//      thread of expert e turns its row of the bitmap into the row of each
//      32-token word (its cursor plus the bits set before the word), and each
//      assignment writes its token at that row plus the bits set below its own
//      in the word -- so row_index lists each expert's tokens ascending, with
//      no dependence on thread timing.
// Segments are dense over all experts (segment e is expert e, possibly empty),
// so the host needs no count back before launching the grouped matmul.
#include <hip/hip_runtime.h>

#include <math.h>

#include "qmm_device.h"
#include "qmm_internal.h"
#include "qmm_launch.h"

namespace qmm {
namespace {

constexpr uint32_t kOOBr = 0x80000000u;   // buffer offset past every range: reads zero

// ---- 1. scores ----
// One workgroup per 32 tokens × 32 experts (2 × 2 blocks of 16 × 16); its
// eight waves take interleaved 64-code pieces of d (wave w: pieces w, w + 8,
// ...).  The MFMA operand layout puts 16 different rows on adjacent lanes,
// which global loads serve poorly (rows are d·2 bytes apart), so each wave
// stages its pieces through a private LDS region: global loads with 8 lanes
// on each row's 128 contiguous bytes, then ds_read_b128 in operand layout.
// The region is the wave's own, so no barrier is needed until the end, where
// waves 0-3 each add the eight partial sums of one block in wave order
// through LDS -- the result does not depend on timing.
//
// Tile order: workgroups are dealt round-robin to the 8 XCDs, and XCD k
// takes one cell of an a × (8/a) split of the token-tile × expert-tile grid
// (a chosen on the host), so each XCD's L2 holds a slice of x and of R
// instead of every XCD streaming all of R.
constexpr int kRT = 32;                 // tokens and experts per workgroup
constexpr int kRWaves = 8;
constexpr int kRPiece = 64;             // codes per piece
constexpr int kRRows = 2 * kRT;         // staged rows per piece: tokens, then experts
constexpr int kRLanesRow = kRPiece * 2 / 16;   // lanes per staged row (16 B each)
constexpr int kRRowsLoad = 64 / kRLanesRow;    // rows per b128 load instruction
constexpr int kRLoads = kRRows / kRRowsLoad;   // b128 loads per lane per piece
constexpr int kRRowLds = 2 * kRPiece + 16;     // padded LDS row (bytes)
constexpr int kRWaveLds = kRRows * kRRowLds;

__global__ __launch_bounds__(64 * kRWaves) void route_scores_kernel(
    const uint16_t* __restrict__ x, int t, int d, const uint16_t* __restrict__ r, int ne,
    float* __restrict__ scores, int tiles_t, int tiles_e, int split_t) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[kRWaves * kRWaveLds];
  // this workgroup's tile: XCD k = id mod 8 owns cell (k mod a, k / a)
  const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
  const int split_e = 8 / split_t;
  const int ct = xcd % split_t, ce = xcd / split_t;
  const int ts = ct * tiles_t / split_t, te_ = (ct + 1) * tiles_t / split_t;
  const int es = ce * tiles_e / split_e, ee_ = (ce + 1) * tiles_e / split_e;
  const int nt = te_ - ts;
  if (local >= nt * (ee_ - es)) return;   // whole workgroup, before any barrier
  const int t0 = (ts + local % nt) * kRT, e0 = (es + local / nt) * kRT;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: loop control stays scalar
  const int col = lane & 15, g = lane >> 4;
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, uint32_t(t) * uint32_t(d) * 2u);
  const __amdgpu_buffer_rsrc_t rr = make_rsrc(r, uint32_t(ne) * uint32_t(d) * 2u);
  // staging: load i covers row kRRowsLoad·i + (lane / kRLanesRow), bytes
  // 16·(lane mod kRLanesRow) .. +15 of the row's piece; rows 0-31 are tokens
  // t0 .., rows 32-63 experts e0 ..
  const int srow = lane / kRLanesRow, sc = lane % kRLanesRow;
  uint32_t rowoff[kRLoads];
#pragma unroll
  for (int i = 0; i < kRLoads; ++i) {
    const int row = kRRowsLoad * i + srow;
    if (i < kRLoads / 2) {
      const int tt = t0 + row;
      rowoff[i] = tt < t ? uint32_t(tt) * uint32_t(d) * 2u : kOOBr;
    } else {
      const int ee = e0 + row - kRT;
      rowoff[i] = ee < ne ? uint32_t(ee) * uint32_t(d) * 2u : kOOBr;
    }
  }
  auto load_piece = [&](u32x4_t (&v)[kRLoads], int piece) {
    const int k = piece * kRPiece + 8 * sc;
    const bool kin = k < d;
#pragma unroll
    for (int i = 0; i < kRLoads; ++i) {
      const uint32_t off = (kin ? rowoff[i] + 2u * uint32_t(k) : kOOBr) | (rowoff[i] & kOOBr);
      v[i] = buf_load16(i < kRLoads / 2 ? xr : rr, off);   // first half: token rows
    }
  };
  unsigned char* my = lds + wave * kRWaveLds;
  const int npieces = (d + kRPiece - 1) / kRPiece;
  f32x4_t acc[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) acc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto stage_and_compute = [&](const u32x4_t (&v)[kRLoads]) {
#pragma unroll
    for (int i = 0; i < kRLoads; ++i)
      *reinterpret_cast<u32x4_t*>(my + (kRRowsLoad * i + srow) * kRRowLds + 16 * sc) = v[i];
#pragma unroll
    for (int u = 0; u < kRPiece / 32; ++u) {
      bf16x8_t a[2], b[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        a[h] = *reinterpret_cast<const bf16x8_t*>(my + (16 * h + col) * kRRowLds + 64 * u + 16 * g);
        b[h] = *reinterpret_cast<const bf16x8_t*>(my + (kRT + 16 * h + col) * kRRowLds + 64 * u + 16 * g);
      }
#pragma unroll
      for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < 2; ++bj)
          acc[2 * bi + bj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[bi], b[bj], acc[2 * bi + bj], 0, 0, 0);
    }
  };
  // Two pieces in flight, one loop shape: a piece past the end loads zeros,
  // which add nothing (at most one such piece is staged per wave).  Loads
  // complete in issue order, so they are issued in the order they are staged
  // (the scheduling barriers keep the scheduler from swapping batches).
  u32x4_t v0[kRLoads], v1[kRLoads];
  load_piece(v0, wave);
  __builtin_amdgcn_sched_barrier(0);
  load_piece(v1, wave + kRWaves);
  for (int p = wave; p < npieces; p += 2 * kRWaves) {
    stage_and_compute(v0);
    load_piece(v0, p + 2 * kRWaves);
    __builtin_amdgcn_sched_barrier(0);
    stage_and_compute(v1);
    load_piece(v1, p + 3 * kRWaves);
    __builtin_amdgcn_sched_barrier(0);
  }
  __syncthreads();   // every wave is done with its staging region
  f32x4_t* part = reinterpret_cast<f32x4_t*>(lds);   // [wave][block][lane]
#pragma unroll
  for (int b = 0; b < 4; ++b) part[(wave * 4 + b) * 64 + lane] = acc[b];
  __syncthreads();
  if (wave >= 4) return;
  // wave w finishes block w: tokens t0 + 16 (w >> 1) + 4g + i, expert e0 + 16 (w & 1) + col
  f32x4_t sum = part[wave * 64 + lane];
#pragma unroll
  for (int w = 1; w < kRWaves; ++w) {
    const f32x4_t q = part[(w * 4 + wave) * 64 + lane];
#pragma unroll
    for (int i = 0; i < 4; ++i) sum[i] += q[i];
  }
  const int e = e0 + 16 * (wave & 1) + col;
  if (e >= ne) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tt = t0 + 16 * (wave >> 1) + 4 * g + i;
    if (tt < t) scores[int64_t(tt) * ne + e] = 1.0f / (1.0f + expf(-sum[i]));
  }
}

// ---- 2. top-k ----
constexpr int kMaxExperts = 1024;
constexpr int kEJ = kMaxExperts / 64;   // scores per lane

// Order-preserving map of a score to an unsigned key, larger ranks first:
// -0 counts as +0, -inf ranks below every finite score and NaN below -inf.
// Key 0 is below all of them and marks an expert taken or past the end.
__device__ __forceinline__ uint32_t rank_key(float s) {
  const uint32_t b = __float_as_uint(s) == 0x80000000u ? 0u : __float_as_uint(s);
  const uint32_t flip = uint32_t(int32_t(b) >> 31) | 0x80000000u;   // negative: all bits
  return s != s ? 1u : (b ^ flip);
}

__device__ __forceinline__ uint32_t dpp_max(uint32_t v) {
  // within each row of 16 lanes: swap pairs, swap pair-pairs, mirror the half
  // row, mirror the row; then the four row results through scalar registers
  v = max(v, uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0xB1, 0xF, 0xF, false)));
  v = max(v, uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x4E, 0xF, 0xF, false)));
  v = max(v, uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x141, 0xF, 0xF, false)));
  v = max(v, uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x140, 0xF, 0xF, false)));
  const uint32_t r0 = __builtin_amdgcn_readlane(int(v), 0), r1 = __builtin_amdgcn_readlane(int(v), 16);
  const uint32_t r2 = __builtin_amdgcn_readlane(int(v), 32), r3 = __builtin_amdgcn_readlane(int(v), 48);
  return max(max(r0, r1), max(r2, r3));
}

__device__ __forceinline__ uint32_t dpp_min(uint32_t v) {
  v = min(v, uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0xB1, 0xF, 0xF, false)));
  v = min(v, uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x4E, 0xF, 0xF, false)));
  v = min(v, uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x141, 0xF, 0xF, false)));
  v = min(v, uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x140, 0xF, 0xF, false)));
  const uint32_t r0 = __builtin_amdgcn_readlane(int(v), 0), r1 = __builtin_amdgcn_readlane(int(v), 16);
  const uint32_t r2 = __builtin_amdgcn_readlane(int(v), 32), r3 = __builtin_amdgcn_readlane(int(v), 48);
  return min(min(r0, r1), min(r2, r3));
}

// One wave per token; lane l holds the keys of experts l, l + 64, ...: the
// selection score fp32(sigmoid + bias) of each.  Each of the k rounds takes
// the largest key, the lowest expert id among equal keys, and zeroes the
// winner's key.  Branch-free: every lane runs every step.
__global__ __launch_bounds__(64) void route_topk_kernel(const float* __restrict__ scores,
                                                        const float* __restrict__ bias, int t,
                                                        int ne, int k, int32_t* __restrict__ topk) {
  const int lane = threadIdx.x;
  const int tok = blockIdx.x;
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(scores + int64_t(tok) * ne, uint32_t(ne) * 4u);
  // no bias: a descriptor of size zero, every load reads zero
  const __amdgpu_buffer_rsrc_t br = make_rsrc(bias ? bias : scores, bias ? uint32_t(ne) * 4u : 0u);
  float v[kEJ];
#pragma unroll
  for (int j = 0; j < kEJ; ++j)   // past the row's end reads zero
    v[j] = __uint_as_float(buf_load4(sr, uint32_t(lane + 64 * j) * 4u)) +
           __uint_as_float(buf_load4(br, uint32_t(lane + 64 * j) * 4u));
  uint32_t key[kEJ];
#pragma unroll
  for (int j = 0; j < kEJ; ++j) {
    const uint32_t kj = rank_key(v[j]);
    key[j] = lane + 64 * j < ne ? kj : 0u;
  }
  int32_t mine = 0;
  for (int r = 0; r < k; ++r) {
    uint32_t bk = key[0], be = uint32_t(lane);
#pragma unroll
    for (int j = 1; j < kEJ; ++j) {   // ascending ids: strictly greater keeps the lower id
      const bool gt = key[j] > bk;
      bk = gt ? key[j] : bk;
      be = gt ? uint32_t(lane + 64 * j) : be;
    }
    const uint32_t m = dpp_max(bk);
    const uint32_t win = dpp_min(bk == m ? be : 0xFFFFFFFFu);
#pragma unroll
    for (int j = 0; j < kEJ; ++j) key[j] = uint32_t(lane + 64 * j) == win ? 0u : key[j];
    mine = lane == r ? int32_t(win) : mine;
  }
  if (lane < k) topk[int64_t(tok) * k + lane] = mine;
}

// ---- 3. grouping ----
constexpr int kGroupBlock = 512;   // tokens per bitmap pass
constexpr int kGroupCache = 16;    // top-k entries a thread holds when t·k <= 1024·16

__global__ __launch_bounds__(1024) void route_group_kernel(const int32_t* __restrict__ topk, int t,
                                                           int ne, int k,
                                                           int32_t* __restrict__ seg_expert,
                                                           int32_t* __restrict__ seg_offsets,
                                                           int32_t* __restrict__ row_index) {
  __shared__ int32_t cnt[kMaxExperts];
  __shared__ uint32_t bits[kMaxExperts][kGroupBlock / 32];
  __shared__ int32_t wrow[kMaxExperts][kGroupBlock / 32];   // row of each word's first set bit
  __shared__ int32_t wsum[16];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int na = t * k;   // below 2^30
  // Small tables (the usual case) are read once, all loads in flight together,
  // and kept in registers for both passes; larger ones are streamed per pass
  // with four loads in flight.  Loads past the end re-read the last entry and
  // are not used.  Ids outside [0, ne) are skipped in the counts and the
  // bitmaps alike, so no cursor can pass its segment's end.
  const bool cached = na <= 1024 * kGroupCache;
  int32_t ent[kGroupCache];
  if (cached) {
#pragma unroll
    for (int u = 0; u < kGroupCache; ++u) ent[u] = topk[min(tid + 1024 * u, na - 1)];
  }
  cnt[tid] = 0;
  __syncthreads();
  if (cached) {
#pragma unroll
    for (int u = 0; u < kGroupCache; ++u)
      if (tid + 1024 * u < na && uint32_t(ent[u]) < uint32_t(ne)) atomicAdd(&cnt[ent[u]], 1);
  } else {
    for (int i0 = tid; i0 < na; i0 += 4096) {
      int32_t e[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) e[u] = topk[min(i0 + 1024 * u, na - 1)];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (i0 + 1024 * u < na && uint32_t(e[u]) < uint32_t(ne)) atomicAdd(&cnt[e[u]], 1);
    }
  }
  __syncthreads();
  // exclusive scan of cnt[0 .. 1024): within waves, then across the 16 waves
  const int c = cnt[tid];
  int incl = c;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int up = __shfl_up(incl, o);
    if (lane >= o) incl += up;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += wsum[w];
  int cursor = before + incl - c;   // this expert's first row
  if (tid < ne) {
    seg_expert[tid] = tid;
    seg_offsets[tid] = cursor;
  }
  if (tid == ne - 1) seg_offsets[ne] = cursor + c;
  // tokens in blocks: mark each assignment's bit, give each 32-token word of
  // an expert its first row, then every assignment writes its own row
  auto place = [&](int e, int il, int b0) {   // assignment il of the block, expert e
    const int tl = il / k, h = tl >> 5;
    const uint32_t below = bits[e][h] & ((1u << (tl & 31)) - 1u);
    row_index[wrow[e][h] + __builtin_popcount(below)] = b0 + tl;
  };
  for (int b0 = 0; b0 < t; b0 += kGroupBlock) {
#pragma unroll
    for (int h = 0; h < kGroupBlock / 32; ++h) bits[tid][h] = 0u;
    __syncthreads();
    const int nb = min(kGroupBlock, t - b0);
    const int nab = nb * k, base = b0 * k;
    if (cached) {
#pragma unroll
      for (int u = 0; u < kGroupCache; ++u) {
        const int il = tid + 1024 * u - base;   // entry index inside this block
        if (il >= 0 && il < nab && uint32_t(ent[u]) < uint32_t(ne)) {
          const int tl = il / k;
          atomicOr(&bits[ent[u]][tl >> 5], 1u << (tl & 31));
        }
      }
    } else {
      for (int i0 = tid; i0 < nab; i0 += 4096) {
        int32_t e[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) e[u] = topk[base + min(i0 + 1024 * u, nab - 1)];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int il = i0 + 1024 * u;
          if (il < nab && uint32_t(e[u]) < uint32_t(ne)) {
            const int tl = il / k;
            atomicOr(&bits[e[u]][tl >> 5], 1u << (tl & 31));
          }
        }
      }
    }
    __syncthreads();
    if (tid < ne) {
#pragma unroll
      for (int h = 0; h < kGroupBlock / 32; ++h) {
        wrow[tid][h] = cursor;
        cursor += __builtin_popcount(bits[tid][h]);
      }
    }
    __syncthreads();
    // a token listed twice for one expert sets one bit: both entries write
    // the same row, and the expert's cursor advances by one
    if (cached) {
#pragma unroll
      for (int u = 0; u < kGroupCache; ++u) {
        const int il = tid + 1024 * u - base;
        if (il >= 0 && il < nab && uint32_t(ent[u]) < uint32_t(ne)) place(ent[u], il, b0);
      }
    } else {
      for (int i0 = tid; i0 < nab; i0 += 4096) {
        int32_t e[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) e[u] = topk[base + min(i0 + 1024 * u, nab - 1)];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int il = i0 + 1024 * u;
          if (il < nab && uint32_t(e[u]) < uint32_t(ne)) place(e[u], il, b0);
        }
      }
    }
    __syncthreads();
  }
}

}  // namespace

int launch_route(const RouteArgs& a, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  // armed profiling events bracket the three launches: start stamped by the
  // first dispatch, stop by the last
  const ProfileEvents pe = take_profile_events();
  const hipEvent_t ev0 = static_cast<hipEvent_t>(pe.start), ev1 = static_cast<hipEvent_t>(pe.stop);
  // XCD split: the a × (8/a) cell grid with the fewest workgroups per XCD,
  // then the fewest rows (bytes of x and R) per XCD
  const int tiles_t = (a.t + kRT - 1) / kRT, tiles_e = (a.ne + kRT - 1) / kRT;
  int split_t = 1;
  int64_t best_cells = -1, best_rows = 0;
  for (int st = 1; st <= 8; st *= 2) {
    const int64_t ct = (tiles_t + st - 1) / st, ce = (tiles_e + 8 / st - 1) / (8 / st);
    if (best_cells < 0 || ct * ce < best_cells || (ct * ce == best_cells && ct + ce < best_rows)) {
      best_cells = ct * ce;
      best_rows = ct + ce;
      split_t = st;
    }
  }
  hipExtLaunchKernelGGL(route_scores_kernel, dim3(unsigned(8 * best_cells)), dim3(64 * kRWaves), 0, s, ev0,
                        nullptr, 0, a.x, a.t, a.d, a.r, a.ne, a.scores, tiles_t, tiles_e, split_t);
  int err = int(hipGetLastError());
  if (err) return err;
  hipLaunchKernelGGL(route_topk_kernel, dim3(unsigned(a.t)), dim3(64), 0, s,
                     static_cast<const float*>(a.scores), a.bias, a.t, a.ne, a.k, a.topk);
  err = int(hipGetLastError());
  if (err) return err;
  hipExtLaunchKernelGGL(route_group_kernel, dim3(1), dim3(1024), 0, s, nullptr, ev1, 0,
                        static_cast<const int32_t*>(a.topk), a.t, a.ne, a.k, a.seg_expert,
                        a.seg_offsets, a.row_index);
  return int(hipGetLastError());
}

}  // namespace qmm
