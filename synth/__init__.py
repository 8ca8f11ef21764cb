"""Seeded synthetic inputs for the 4-bit weight-quantized matmul Y = X·Wᵀ.

This module produces the *canonical* inputs that both the HIP path and the CPU
oracle consume: packed 4-bit codes, bf16 scales/biases or E8M0 exponents, bf16
activations, and the MoE routing tables of the prefill workload.  It holds none
of the matmul's arithmetic (no dequantisation, no dot products): only counter
hashing, the value distributions, and bf16/fp32 rounding of generated numbers.

Counter-based generator
-----------------------
Every integer comes from SplitMix64's output function (Steele, Lea & Flood,
"Fast splittable pseudorandom number generators", OOPSLA 2014; the constants
are those of Vigna's public-domain reference code), used in counter mode::

    key(seed, stream, sub) = mix64((seed << 32) ^ (stream << 20) ^ sub ^ K0)
    h(seed, stream, sub, i) = mix64(key + (i + 1) * GAMMA)        (mod 2**64)

so any element can be regenerated on its own, on the host (numpy, here) or on
the GPU (``synth/csrc/synth_gen.hip``), bit for bit.  ``seed`` < 2**32,
``stream`` < 2**12, ``sub`` < 2**20.

Derived values:

* code bytes: the byte stream of h(i) for i = 0, 1, ... (little endian, eight
  bytes per hash).  Every nibble is uniform over 0..15.  Affine code words
  (uint32, eight codes each) and MXFP4 code bytes (two codes each) are both
  read from this stream.
* uniform in [0, 1): (h >> 11) * 2**-53.
* small integer in [lo, lo + m): lo + (((h >> 32) * m) >> 32).
* N(0, 1): Box–Muller on the pair of uniforms u1 = U(2j), u2 = U(2j + 1) for
  elements 2j and 2j + 1: r = sqrt(-2 ln(1 - u1)); cos branch for the even
  element, sin branch for the odd one.
* bf16: fp64 -> fp32 -> bf16, each step round-to-nearest-even.  The bits so
  produced *are* the input both sides read, so the route only has to be fixed,
  not to equal a single rounding of the fp64 value.

Streams: 1 affine codes, 2 scales, 3 biases, 4 x / X, 5 z, 6 router weights R,
7 router bias, 8 expert draw, 11/12 gate_up codes/E8M0, 13/14 down codes/E8M0.
"""
from __future__ import annotations

import dataclasses
import hashlib

import numpy as np

MASK64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15
M1 = 0xBF58476D1CE4E5B9
M2 = 0x94D049BB133111EB
K0 = 0x243F6A8885A308D3

S_CODES, S_SCALE, S_BIAS, S_X, S_Z, S_R, S_RBIAS, S_DRAW = 1, 2, 3, 4, 5, 6, 7, 8
S_GU_CODES, S_GU_E8M0, S_DN_CODES, S_DN_E8M0 = 11, 12, 13, 14


def _mix64_int(z: int) -> int:
    z &= MASK64
    z = ((z ^ (z >> 30)) * M1) & MASK64
    z = ((z ^ (z >> 27)) * M2) & MASK64
    return z ^ (z >> 31)


def key(seed: int, stream: int, sub: int = 0) -> int:
    if not (0 <= seed < 1 << 32 and 0 <= stream < 1 << 12 and 0 <= sub < 1 << 20):
        raise ValueError("seed/stream/sub out of range")
    return _mix64_int((seed << 32) ^ (stream << 20) ^ sub ^ K0)


def _mix64(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * np.uint64(M1)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(M2)
        return z ^ (z >> np.uint64(31))


def hashes(seed: int, stream: int, sub: int, start: int, count: int) -> np.ndarray:
    """h(seed, stream, sub, i) for i in [start, start + count) as uint64."""
    k = np.uint64(key(seed, stream, sub))
    i = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix64(k + i * np.uint64(GAMMA))


def hashes_at(seed: int, stream: int, sub: int, idx) -> np.ndarray:
    """h(seed, stream, sub, i) for every i in the integer array `idx`."""
    k = np.uint64(key(seed, stream, sub))
    i = np.asarray(idx, np.uint64) + np.uint64(1)
    with np.errstate(over="ignore"):
        return _mix64(k + i * np.uint64(GAMMA))


def code_bytes(seed: int, stream: int, sub: int, nbytes: int, start_byte: int = 0) -> np.ndarray:
    """Bytes [start_byte, start_byte + nbytes) of the little-endian hash stream."""
    if nbytes == 0:
        return np.zeros(0, np.uint8)
    h0 = start_byte // 8
    h1 = (start_byte + nbytes + 7) // 8
    raw = hashes(seed, stream, sub, h0, h1 - h0).astype("<u8").view(np.uint8)
    off = start_byte - 8 * h0
    return raw[off:off + nbytes].copy()


def uniform(seed: int, stream: int, sub: int, count: int, start: int = 0) -> np.ndarray:
    h = hashes(seed, stream, sub, start, count)
    return (h >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def small_int(seed: int, stream: int, sub: int, count: int, lo: int, m: int, start: int = 0) -> np.ndarray:
    h = hashes(seed, stream, sub, start, count)
    return (lo + (((h >> np.uint64(32)) * np.uint64(m)) >> np.uint64(32))).astype(np.int64)


def normal(seed: int, stream: int, sub: int, count: int) -> np.ndarray:
    npair = (count + 1) // 2
    u = uniform(seed, stream, sub, 2 * npair)
    u1, u2 = u[0::2], u[1::2]
    r = np.sqrt(-2.0 * np.log1p(-u1))
    out = np.empty(2 * npair, np.float64)
    out[0::2] = r * np.cos(2.0 * np.pi * u2)
    out[1::2] = r * np.sin(2.0 * np.pi * u2)
    return out[:count]


def bf16_bits(v: np.ndarray) -> np.ndarray:
    """fp64 -> bf16 bit patterns (uint16), round to nearest even."""
    f = np.asarray(v, np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    rounded = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return rounded.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# --------------------------------------------------------------------------
# Canonical tensors
# --------------------------------------------------------------------------

@dataclasses.dataclass
class Affine:
    """Canonical affine 4-bit weights W[N, D]: codes uint32[N, D/8] (code k of a
    row is nibble k % 8 of word k // 8, lowest nibble first), scale and bias as
    bf16 bit patterns uint16[N, D/64]."""
    codes: np.ndarray
    scale: np.ndarray
    bias: np.ndarray

    @property
    def n(self) -> int:
        return self.codes.shape[0]

    @property
    def d(self) -> int:
        return self.codes.shape[1] * 8


@dataclasses.dataclass
class MXFP4:
    """Canonical MXFP4 weights W[N, D]: codes uint8[N, D/2] (element k in byte
    k // 2, low nibble for even k), E8M0 exponents uint8[N, D/32]."""
    codes: np.ndarray
    e8m0: np.ndarray

    @property
    def n(self) -> int:
        return self.codes.shape[0]

    @property
    def d(self) -> int:
        return self.codes.shape[1] * 2


def affine_weights(seed: int, n: int, d: int) -> Affine:
    """Codes uniform in 0..15; scale ~U[0.01, 0.05]; bias ~U[-0.4, 0] per group of 64."""
    if d % 64:
        raise ValueError("d must be a multiple of 64")
    codes = code_bytes(seed, S_CODES, 0, n * d // 2).view("<u4").reshape(n, d // 8)
    g = n * (d // 64)
    scale = bf16_bits(0.01 + 0.04 * uniform(seed, S_SCALE, 0, g)).reshape(n, d // 64)
    bias = bf16_bits(-0.4 * uniform(seed, S_BIAS, 0, g)).reshape(n, d // 64)
    return Affine(codes.astype(np.uint32), scale, bias)


def mxfp4_weights(seed: int, n: int, d: int, codes_stream: int, e8m0_stream: int, sub: int,
                  e_lo: int = 118, e_count: int = 9) -> MXFP4:
    """Codes uniform over the 16 E2M1 patterns; E8M0 uniform in [e_lo, e_lo + e_count)."""
    if d % 32:
        raise ValueError("d must be a multiple of 32")
    codes = code_bytes(seed, codes_stream, sub, n * d // 2).reshape(n, d // 2)
    e = small_int(seed, e8m0_stream, sub, n * (d // 32), e_lo, e_count).astype(np.uint8)
    return MXFP4(codes, e.reshape(n, d // 32))


def mxfp4_rows(seed: int, n: int, d: int, codes_stream: int, e8m0_stream: int, sub: int, rows,
               e_lo: int = 118, e_count: int = 9) -> MXFP4:
    """Rows `rows` of mxfp4_weights(seed, n, d, ...), each regenerated on its
    own from its place in the counter streams (row j's codes are bytes
    [j·d/2, (j+1)·d/2) of the code stream, its exponents elements
    [j·d/32, (j+1)·d/32) of the E8M0 stream)."""
    rows = np.asarray(rows, np.int64).reshape(-1)
    if d % 32 or rows.size and (rows.min() < 0 or rows.max() >= n):
        raise ValueError("d must be a multiple of 32 and rows inside [0, n)")
    b = rows[:, None] * (d // 2) + np.arange(d // 2)[None, :]          # byte offsets in the code stream
    h = hashes_at(seed, codes_stream, sub, b // 8)
    codes = ((h >> (np.uint64(8) * (b % 8).astype(np.uint64))) & np.uint64(0xFF)).astype(np.uint8)
    ie = rows[:, None] * (d // 32) + np.arange(d // 32)[None, :]
    he = hashes_at(seed, e8m0_stream, sub, ie)
    e = e_lo + (((he >> np.uint64(32)) * np.uint64(e_count)) >> np.uint64(32)).astype(np.int64)
    return MXFP4(codes, e.astype(np.uint8))


def expert_gate_up_rows(seed: int, e: int, rows, n: int = 6144, d: int = 3584) -> MXFP4:
    return mxfp4_rows(seed, n, d, S_GU_CODES, S_GU_E8M0, e, rows)


def expert_gate_up(seed: int, e: int, n: int = 6144, d: int = 3584) -> MXFP4:
    return mxfp4_weights(seed, n, d, S_GU_CODES, S_GU_E8M0, e)


def expert_down(seed: int, e: int, n: int = 3584, d: int = 3072) -> MXFP4:
    return mxfp4_weights(seed, n, d, S_DN_CODES, S_DN_E8M0, e)


def activations(seed: int, stream: int, t: int, d: int, sub: int = 0) -> np.ndarray:
    """bf16 ~N(0, 1) activations as bit patterns uint16[t, d]."""
    return bf16_bits(normal(seed, stream, sub, t * d)).reshape(t, d)


def draw_experts(seed: int, count: int = 16, total: int = 896, sub: int = 0) -> np.ndarray:
    """`count` distinct experts, uniformly, by a partial Fisher–Yates shuffle."""
    perm = np.arange(total, dtype=np.int64)
    h = hashes(seed, S_DRAW, sub, 0, count)
    for i in range(count):
        j = i + int(((int(h[i]) >> 32) * (total - i)) >> 32)
        perm[i], perm[j] = perm[j], perm[i]
    return perm[:count].copy()


def router_inputs(seed: int, t: int = 512, d: int = 3584, experts: int = 896):
    """X bf16 ~N(0,1)[t, d]; R bf16 ~N(0, 0.02)[experts, d]; bias fp32 ~U[-0.1, 0.1]."""
    x = activations(seed, S_X, t, d)
    r = bf16_bits(0.02 * normal(seed, S_R, 0, experts * d)).reshape(experts, d)
    b = (-0.1 + 0.2 * uniform(seed, S_RBIAS, 0, experts)).astype(np.float32)
    return x, r, b


def sha256(*arrays: np.ndarray) -> str:
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


# --------------------------------------------------------------------------
# The five workloads (seed = 1000 + index)
# --------------------------------------------------------------------------

CONFIGS = {
    0: dict(name="affine4_g64_gemv_T1_D256_N512", kind="gemv", fmt="affine", t=1, d=256, n=512),
    1: dict(name="affine4_g64_gemv_T1_D5120_N13824", kind="gemv", fmt="affine", t=1, d=5120, n=13824),
    2: dict(name="affine4_g64_gemm_T2048_D5120_N13824", kind="gemm", fmt="affine", t=2048, d=5120, n=13824),
    3: dict(name="mxfp4_g32_moe_decode_grouped_gemv_E896_top16", kind="moe_decode", fmt="mxfp4",
            experts=896, top=16, gu_n=6144, gu_d=3584, dn_n=3584, dn_d=3072),
    4: dict(name="mxfp4_g32_moe_prefill_grouped_gemm_T512_E896_top16", kind="moe_prefill", fmt="mxfp4",
            experts=896, top=16, t=512, gu_n=6144, gu_d=3584),
}


def seed_of(cfg: int) -> int:
    return 1000 + cfg
