// Device helpers for the gfx950 kernels: bf16 packing, cross-lane reduction,
// and the in-register dequantisation of the two 4-bit formats.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmm {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float(uint32_t(v) << 16); }

// fp32 -> bf16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return uint16_t((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// Two fp32 -> one register of two bf16 (lo in the low half), RNE.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// 2-wide bf16 dot product accumulated in fp32: acc + a.lo*b.lo + a.hi*b.hi.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), acc, false);
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over each aligned group of 16 lanes; every lane of the group gets it.
// Order is fixed: pairs, quads, half-rows, rows.
__device__ __forceinline__ float sum16(float v) {
  v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f<0x141>(v);  // row_half_mirror
  v += dpp_f<0x140>(v);  // row_mirror
  return v;
}

// ---------------------------------------------------------------------------
// Affine: 32 codes (four device words, see qmm_internal.h) against 32
// activations held as 16 bf16 pairs.  The nibble pair of each shift lands in
// the mantissa of the bf16 constant 128.0 (0x4300), giving 128 + q exactly,
// so the dot yields Σ x·(128 + q) and the caller removes 128·Σx.
// ---------------------------------------------------------------------------
constexpr uint32_t kMagic128x2 = 0x43004300u;

// (a & mask) | magic in one VOP3 instruction.  gfx9 VOP3 cannot encode a
// 32-bit literal, so left to itself the compiler splits this into an AND and
// an OR with literals; here the mask sits in an SGPR and the magic in a VGPR.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t magic) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(mask), "v"(magic));
  return r;
}

// Four independent accumulator chains (one per word) keep the dot unit busy
// without relying on other waves to hide its latency.
__device__ __forceinline__ float affine_dot32(const u32x4_t w, const uint32_t* xp) {
  const uint32_t mask = 0x000F000Fu, magic = kMagic128x2;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int sh = 0; sh < 4; ++sh)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc[i] = dot2_bf16(and_or(w[i] >> (4 * sh), mask, magic), xp[4 * i + sh], acc[i]);
  return (acc[0] + acc[1]) + (acc[2] + acc[3]);
}

// MXFP4: 32 codes (16 bytes) against 32 activations, E2M1 values unscaled
// (the conversion's scale operand is 1.0); the caller applies 2^(E-127).
__device__ __forceinline__ float mxfp4_dot32(const u32x4_t w, const uint32_t* xp) {
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
#define QMM_FP4_STEP(SEL)                                                                 \
  _Pragma("unroll") for (int i = 0; i < 4; ++i) acc[i] = dot2_bf16(                       \
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], 1.0f, SEL)), \
      xp[4 * i + SEL], acc[i]);
  QMM_FP4_STEP(0)
  QMM_FP4_STEP(1)
  QMM_FP4_STEP(2)
  QMM_FP4_STEP(3)
#undef QMM_FP4_STEP
  return (acc[0] + acc[1]) + (acc[2] + acc[3]);
}

// ---------------------------------------------------------------------------
// MFMA B-operand dequantisation: one device word (8 consecutive codes) to
// eight bf16 weights in k order, packed as 4 registers.
// ---------------------------------------------------------------------------

// Affine: w = s·q + b in fp32 (exact), rounded once to bf16.
// Word bytes after masking: lo = (q0, q4, q1, q5), hi = (q2, q6, q3, q7).
__device__ __forceinline__ u32x4_t affine_word_to_bf16x8(uint32_t v, float s, float b) {
  const uint32_t lo = v & 0x0F0F0F0Fu;
  const uint32_t hi = (v >> 4) & 0x0F0F0F0Fu;
  // (float)((v >> 8k) & 0xFF) selects v_cvt_f32_ubyte{k}: one instruction per code
  const float q0 = float(lo & 0xFFu), q4 = float((lo >> 8) & 0xFFu);
  const float q1 = float((lo >> 16) & 0xFFu), q5 = float(lo >> 24);
  const float q2 = float(hi & 0xFFu), q6 = float((hi >> 8) & 0xFFu);
  const float q3 = float((hi >> 16) & 0xFFu), q7 = float(hi >> 24);
  u32x4_t r;
  r[0] = pack_bf16x2(__builtin_fmaf(s, q0, b), __builtin_fmaf(s, q1, b));
  r[1] = pack_bf16x2(__builtin_fmaf(s, q2, b), __builtin_fmaf(s, q3, b));
  r[2] = pack_bf16x2(__builtin_fmaf(s, q4, b), __builtin_fmaf(s, q5, b));
  r[3] = pack_bf16x2(__builtin_fmaf(s, q6, b), __builtin_fmaf(s, q7, b));
  return r;
}

// Affine, MFMA path: the same w = s·q + b with one instruction per weight.
// Masking a nibble pair into the two halves of a register makes two fp16
// subnormals q·2^-24 (nibbles at bits 0..3 of each half) or q·2^-20 (bits
// 4..7), and v_fma_mix_f32 then forms s'·(fp16) + b in fp32 with one rounding,
// where s' = s·2^24 or s·2^20 (exact while finite; qmm_pack rejects scales of
// magnitude 2^100 or more).  The result equals fmaf(s, q, b) bit for bit.
struct AffineMix {
  float s24, s20, b;
};
__device__ __forceinline__ AffineMix affine_mix_consts(uint32_t m) {
  const float s = bf16_lo(m);
  return {s * 16777216.0f, s * 1048576.0f, bf16_hi(m)};
}
__device__ __forceinline__ float f16_lo(uint32_t v) {
  return float(__builtin_bit_cast(_Float16, uint16_t(v)));
}
__device__ __forceinline__ float f16_hi(uint32_t v) {
  return float(__builtin_bit_cast(_Float16, uint16_t(v >> 16)));
}
__device__ __forceinline__ u32x4_t affine_word_to_bf16x8_mix(uint32_t v, const AffineMix& c) {
  const uint32_t v8 = v >> 8;
  const uint32_t p0 = v & 0x000F000Fu, p1 = v & 0x00F000F0u;    // (q0, q1), (q2, q3)
  const uint32_t p2 = v8 & 0x000F000Fu, p3 = v8 & 0x00F000F0u;  // (q4, q5), (q6, q7)
  u32x4_t r;
  r[0] = pack_bf16x2(__builtin_fmaf(c.s24, f16_lo(p0), c.b), __builtin_fmaf(c.s24, f16_hi(p0), c.b));
  r[1] = pack_bf16x2(__builtin_fmaf(c.s20, f16_lo(p1), c.b), __builtin_fmaf(c.s20, f16_hi(p1), c.b));
  r[2] = pack_bf16x2(__builtin_fmaf(c.s24, f16_lo(p2), c.b), __builtin_fmaf(c.s24, f16_hi(p2), c.b));
  r[3] = pack_bf16x2(__builtin_fmaf(c.s20, f16_lo(p3), c.b), __builtin_fmaf(c.s20, f16_hi(p3), c.b));
  return r;
}

// 2^(e - 127) as fp32 for an E8M0 byte e in [0, 254] (e = 0 is the subnormal 2^-127).
__device__ __forceinline__ float e8m0_scale(uint32_t e) {
  return e ? __uint_as_float(e << 23) : __uint_as_float(0x00400000u);
}

// MXFP4: E2M1(c)·scale converted straight to bf16, exact while the product
// is a normal bf16: for every code when E8M0 is in [2, 252].  At 253 the codes
// of magnitude 4 and 6, at 254 those of magnitude 2 and up, reach 2^128 and
// become ±inf (the GEMV paths scale the fp32 chunk sum instead and may stay
// finite there).
__device__ __forceinline__ u32x4_t mxfp4_word_to_bf16x8(uint32_t v, float scale) {
  u32x4_t r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 0));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 1));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 2));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 3));
  return r;
}

__device__ __forceinline__ u32x4_t load16(const void* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

// Raw buffer resource over [base, base + bytes): loads take a 32-bit byte
// offset, and any dword outside the range reads as zero instead of faulting.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(bytes), 0x00020000);
}
__device__ __forceinline__ u32x4_t buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, int(off), 0, 0));
}
__device__ __forceinline__ uint32_t buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, int(off), 0, 0);
}
__device__ __forceinline__ uint32_t buf_load1(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, int(off), 0, 0);
}

}  // namespace qmm
