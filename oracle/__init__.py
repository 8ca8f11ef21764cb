"""CPU oracle for the 4-bit weight-quantized matmul Y = X·Wᵀ — TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never calls it and shares no code with it: this file has its
own bf16 decoding, nibble extraction, E2M1/E8M0 decoding and rounding.

Everything here is the plain definition evaluated in fp64 with numpy: weights
are dequantised exactly (every affine and MXFP4 weight is a dyadic rational with
few significant bits, so fp64 holds it without rounding) and the contraction is
a library fp64 matmul.  The GPU reaches the same mathematical result in a
different summation order and in fp32, which is why parity is a per-element
tolerance and not bit equality ("优化 kernel 后，要检查请求耗时与数值结果",
Kapitsa 源码拆解 02：权重、矩阵与 Metal: a different K reduction order is expected
to change the last bits and is not an error).

Pins (tests/test_oracle.py): the affine worked example, the 36-byte group size,
the E2M1 value set, exact-rational brute force on tiny shapes, integer-exact
cases, one-hot columns, row sums and the tolerance checker's self-test; for the
router, hand-worked scores and selections on tiny inputs (bias that changes the
choice, ties to the lower id), a naive per-token full sort, the grouping's
invariants and literal tables, and the top-k checker's self-test; for the expert
FFN, hand-worked SiLU values and identities, a literal SwiGLU split, the
SwiGLU tolerance hand-worked and checked to bound every corner of its
interval, and a hand-worked renormalised combine; for the
deferred-dequantisation GEMV, a hand-worked quantisation (half-even ties, the
absmax scale), an integer-exact case and a per-element brute force of both y
and the size of its terms; for the router's fp32 score bound, hand-worked
values and a simulation of fp32 summation in the GPU's order that it must
contain.  No function here is parity-unpinned.
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# Scalar formats
# ---------------------------------------------------------------------------


def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit pattern -> its exact value: the bf16 is the top half of an fp32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(v) -> np.ndarray:
    """Round fp64 to the nearest bf16 (ties to even), returning bit patterns.

    Used only to state the expected bits of results that are exactly
    representable (integer-exact cases); the value is rounded directly from
    fp64 with frexp/ldexp, independent of fp32."""
    v = np.asarray(v, dtype=np.float64)
    out = np.zeros(v.shape, np.uint16)
    flat, res = v.reshape(-1), out.reshape(-1)
    for i, x in enumerate(flat):
        if x == 0.0:
            res[i] = 0x8000 if np.signbit(x) else 0
            continue
        sign = 0x8000 if x < 0 else 0
        m, e = np.frexp(abs(x))            # abs(x) = m * 2**e, m in [0.5, 1)
        q = np.round(np.ldexp(m, 8))       # 8 significant bits, ties to even
        if q == 256:
            q, e = 128.0, e + 1
        exp_field = e - 1 + 127            # value = (q/128) * 2**(e-1)
        if exp_field >= 255:
            res[i] = sign | 0x7F80
        elif exp_field <= 0:                 # subnormal bf16
            q = np.round(np.ldexp(abs(x), 133))
            res[i] = sign | int(q)
        else:
            res[i] = sign | (exp_field << 7) | (int(q) - 128)
    return out


def round_to_bf16(v) -> np.ndarray:
    """Values of fp64 numbers rounded to the nearest bf16 (ties to even),
    vectorised: 8 significant bits for normal numbers, steps of 2**-133 below
    2**-126, overflow to ±inf at (2 - 2**-8)·2**127 and above."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    m, e = np.frexp(a)                              # a = m·2**e, m in [0.5, 1)
    normal = np.ldexp(np.round(np.ldexp(m, 8)), e - 8)
    sub = np.ldexp(np.round(np.ldexp(a, 133)), -133)
    r = np.where(a < 2.0 ** -126, sub, normal)
    r = np.where(r >= 2.0 ** 128, np.inf, r)
    r = np.where(np.isnan(v), np.nan, r)
    return np.copysign(r, v)


def e2m1_value(code) -> np.ndarray:
    """Decode 4-bit E2M1 codes (sign, 2 exponent bits with bias 1, 1 mantissa bit).

    The pages name the format only as "MXFP4: W4, group 32 + E8M0 scale, 4.25
    bit" (Kimi K3 迁移到 Google TPU 的可行性评估, §2 模型解剖, quantisation row);
    the element encoding is that of the OCP Microscaling Formats v1.0
    specification: exponent field 0 is subnormal (value = m/2), otherwise
    2**(e-1) * (1 + m/2); bit 3 is the sign."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where((c >> 3) & 1, -1.0, 1.0)
    e = (c >> 1) & 3
    m = (c & 1).astype(np.float64)
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, (e - 1).astype(np.int64)))
    return sign * mag


def e8m0_value(e) -> np.ndarray:
    """E8M0 shared exponent: 2**(E - 127); E = 255 encodes NaN."""
    e = np.asarray(e, dtype=np.int64)
    return np.where(e == 255, np.nan, np.ldexp(1.0, e - 127))


# ---------------------------------------------------------------------------
# Dequantisation
# ---------------------------------------------------------------------------


def affine_codes(codes_u32) -> np.ndarray:
    """Unsigned 4-bit codes q[N, D] from uint32 words[N, D/8].

    Eight codes share one 32-bit word and are taken out by shift and mask
    (Kapitsa 源码拆解 02, §"权重怎样存储": wf_extract/wf_codes16); code k of a
    row is nibble k % 8 of word k // 8, lowest nibble first (reading: the page
    does not state the nibble order)."""
    w = np.asarray(codes_u32, dtype=np.uint32)
    shifts = (4 * np.arange(8, dtype=np.uint32))
    q = (w[:, :, None] >> shifts[None, None, :]) & np.uint32(0xF)
    return q.reshape(w.shape[0], w.shape[1] * 8).astype(np.int64)


def dequant_affine(codes_u32, scale_bits, bias_bits) -> np.ndarray:
    """Ŵ[n, k] = scale[n, k//64] * q[n, k] + bias[n, k//64], exactly, in fp64.

    Affine format with groups of 64 codes along D, one bf16 scale and one bf16
    bias per group (Kapitsa 源码拆解 02, §"权重怎样存储": w ≈ scale×q + bias)."""
    q = affine_codes(codes_u32).astype(np.float64)
    n, d = q.shape
    if d % 64:
        raise ValueError("D must be a multiple of 64")
    s = np.repeat(bf16_to_f64(scale_bits).reshape(n, d // 64), 64, axis=1)
    b = np.repeat(bf16_to_f64(bias_bits).reshape(n, d // 64), 64, axis=1)
    return s * q + b


def mxfp4_codes(codes_u8) -> np.ndarray:
    """4-bit codes c[N, D] from bytes[N, D/2]: element k is in byte k // 2, low
    nibble for even k (reading: the checkpoint stores MXFP4 "packed as U8",
    Kimi K3 迁移到 Google TPU 的可行性评估, §3.1 权重账)."""
    b = np.asarray(codes_u8, dtype=np.uint8).astype(np.int64)
    c = np.stack([b & 0xF, b >> 4], axis=-1)
    return c.reshape(b.shape[0], b.shape[1] * 2)


def dequant_mxfp4(codes_u8, e8m0) -> np.ndarray:
    """Ŵ[n, k] = E2M1(c[n, k]) * 2**(E[n, k//32] - 127), exactly, in fp64.

    Groups of 32 codes along D share one E8M0 exponent (Kimi K3 迁移到 Google TPU
    的可行性评估, §2 模型解剖: "W4 group 32 + E8M0 scale")."""
    v = e2m1_value(mxfp4_codes(codes_u8))
    n, d = v.shape
    if d % 32:
        raise ValueError("D must be a multiple of 32")
    scale = np.repeat(e8m0_value(np.asarray(e8m0).reshape(n, d // 32)), 32, axis=1)
    return v * scale


# ---------------------------------------------------------------------------
# The contraction
# ---------------------------------------------------------------------------


def matmul(x_bits, w_hat) -> tuple[np.ndarray, np.ndarray]:
    """Y = X·Ŵᵀ and A = |X|·|Ŵ|ᵀ in fp64.

    Row-vector convention X[T, D], W[N, D] (one output feature per row of W),
    Y[T, N] (Kapitsa 源码拆解 02, §"矩阵乘法中数据和参数").  A[t, n] = Σ_k
    |x[t,k]·ŵ[n,k]| is the scale of the tolerance."""
    x = bf16_to_f64(x_bits)
    if x.ndim == 1:
        x = x[None, :]
    w = np.asarray(w_hat, np.float64)
    if x.shape[1] != w.shape[1]:
        raise ValueError("X and W disagree on D")
    return x @ w.T, np.abs(x) @ np.abs(w).T


def gemm_affine(x_bits, codes_u32, scale_bits, bias_bits):
    """Affine decode GEMV (T = 1) and prefill GEMM: Y = X·Ŵᵀ."""
    return matmul(x_bits, dequant_affine(codes_u32, scale_bits, bias_bits))


def gemm_mxfp4(x_bits, codes_u8, e8m0):
    """MXFP4 GEMV/GEMM: Y = X·Ŵᵀ."""
    return matmul(x_bits, dequant_mxfp4(codes_u8, e8m0))


# ---------------------------------------------------------------------------
# Deferred dequantisation (approximate: the activations are quantised to int8)
# ---------------------------------------------------------------------------

def quantize_rows_int8(x_bits):
    """Per-row absmax quantisation of bf16 activations to int8 ("LLM Decode /
    Prefill 优化案例（Metal）", Step 2: the input is quantised per row by its
    absolute maximum before the integer GEMV).  Readings where the page is
    silent: s = fp32(absmax)/127 and x_q = round-half-even(x/s), both in fp32
    (the GPU takes the same decision in the same precision, so the codes match
    exactly); an all-zero row has s = 0 and x_q = 0.  Returns (x_q int64[T, D],
    s float32[T])."""
    x = bf16_to_f64(x_bits).astype(np.float32)
    x = x.reshape(-1, x.shape[-1])
    amax = np.max(np.abs(x), axis=1)
    s = (amax / np.float32(127.0)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    q = np.rint((x / safe[:, None]).astype(np.float32))
    q = np.where(s[:, None] > 0, q, 0.0)
    return q.astype(np.int64), s


def gemv_affine_deferred(x_bits, codes_u32, scale_bits, bias_bits):
    """The deferred-dequantisation decode GEMV of "LLM Decode / Prefill 优化案例
    （Metal）", Step 2, for one activation row: the weights' 4-bit codes meet the
    int8 activations in an exact integer sum per group of 64,
    isum[n, g] = Σ_{k∈g} x_q[k]·q[n, k], and the scales are applied once per
    group afterwards, with the bias corrected through the sum of the quantised
    inputs: y[n] = s_x·Σ_g (scale[n, g]·isum[n, g] + bias[n, g]·Σ_{k∈g} x_q[k]).
    Integer parts exact (int64), the rest in fp64.  Returns (y[N], A[N]) with
    A = s_x·Σ_g (|scale·isum| + |bias·xsum|), the size of the terms."""
    xq, sx = quantize_rows_int8(x_bits)
    xq, sx = xq[0], float(sx[0])
    q = affine_codes(codes_u32)
    n, d = q.shape
    g = d // 64
    isum = (q.reshape(n, g, 64) * xq.reshape(1, g, 64)).sum(axis=2)
    xsum = xq.reshape(g, 64).sum(axis=1)
    sc = bf16_to_f64(scale_bits).reshape(n, g)
    bi = bf16_to_f64(bias_bits).reshape(n, g)
    t1 = sc * isum.astype(np.float64)
    t2 = bi * xsum[None, :].astype(np.float64)
    y = sx * (t1 + t2).sum(axis=1)
    a = sx * (np.abs(t1) + np.abs(t2)).sum(axis=1)
    return y, a


def grouped(x_bits, row_index, seg_expert, seg_offsets, expert_weights, segments=None):
    """Routed-expert grouped matmul, one product per segment.

    Segment s applies expert seg_expert[s] to the activation rows
    X[row_index[r]] for r in [seg_offsets[s], seg_offsets[s+1]) and writes
    rows r of the grouped output (the per-expert GEMM of the MoE block,
    Colibri Kimi K3 Metal 后端实现全解析, Phase 6).  `expert_weights(e)` returns
    the fp64 Ŵ of expert e.  With `segments` given only those segments are
    evaluated; the other output rows are NaN."""
    x_bits = np.asarray(x_bits)
    row_index = np.asarray(row_index)
    seg_offsets = np.asarray(seg_offsets)
    segs = range(len(seg_expert)) if segments is None else segments
    y = a = None
    for s in segs:
        r0, r1 = int(seg_offsets[s]), int(seg_offsets[s + 1])
        if r1 == r0:
            continue
        w = expert_weights(int(seg_expert[s]))
        if y is None:
            m_total = int(seg_offsets[-1])
            y = np.full((m_total, w.shape[0]), np.nan)
            a = np.full((m_total, w.shape[0]), np.nan)
        ys, as_ = matmul(x_bits[row_index[r0:r1]], w)
        y[r0:r1], a[r0:r1] = ys, as_
    return y, a


def sampled(x_bits, w_row, pairs):
    """y[t, n] and A[t, n] for chosen (t, n) pairs only, each as its own dot
    product over k: Σ_k x[t,k]·ŵ[n,k].  `w_row(n)` returns row n of Ŵ in fp64."""
    x = bf16_to_f64(x_bits)
    if x.ndim == 1:
        x = x[None, :]
    y = np.empty(len(pairs))
    a = np.empty(len(pairs))
    cache = {}
    for i, (t, n) in enumerate(pairs):
        if n not in cache:
            cache[n] = w_row(n)
        prod = x[t] * cache[n]
        y[i] = prod.sum()
        a[i] = np.abs(prod).sum()
    return y, a


# ---------------------------------------------------------------------------
# Router (MoE prefill): scores, top-k, tokens grouped by expert
# ---------------------------------------------------------------------------

def route_scores(x_bits, r_bits, bias):
    """score[t, e] = sigmoid(Σ_j x[t,j]·R[e,j]) + bias[e] in fp64, and
    A[t, e] = Σ_j |x[t,j]·R[e,j]| (the size of the logit's terms, for the
    error bound of an fp32 evaluation).

    A sigmoid router whose per-expert bias only corrects the selection (the
    router with a score-correction bias of Colibri Kimi K3 Metal 后端实现全解析,
    introduction; sigmoid scoring with 896 routed experts, top-16, in
    Kimi K3 迁移到 Google TPU 的可行性评估（v2）, §2 模型解剖)."""
    x = bf16_to_f64(x_bits)
    r = bf16_to_f64(r_bits)
    logits = x @ r.T
    a = np.abs(x) @ np.abs(r).T
    b = np.zeros(r.shape[0]) if bias is None else np.asarray(bias, np.float64)
    return 1.0 / (1.0 + np.exp(-logits)) + b[None, :], a


def topk(scores, k):
    """The k experts of each token by score, highest first; equal scores go
    to the lower expert id.  int64[T, k]."""
    scores = np.asarray(scores, np.float64)
    t, e = scores.shape
    order = np.lexsort((np.broadcast_to(np.arange(e), scores.shape), -scores), axis=1)
    return order[:, :k].astype(np.int64)


def group(topk_ids, n_experts):
    """Tokens grouped by expert: segment e (one per expert, possibly empty)
    covers rows [seg_offsets[e], seg_offsets[e+1]) of the grouped order, and
    row r of that order reads token row_index[r]; inside a segment tokens
    ascend.  Returns (seg_offsets int32[E + 1], row_index int32[T·k])."""
    topk_ids = np.asarray(topk_ids)
    t, k = topk_ids.shape
    pairs_e = topk_ids.reshape(-1)
    pairs_t = np.repeat(np.arange(t), k)
    o = np.lexsort((pairs_t, pairs_e))
    counts = np.bincount(pairs_e, minlength=n_experts)
    seg_offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    return seg_offsets, pairs_t[o].astype(np.int32)


class Routing:
    """Grouped-expert tables with the empty segments dropped (segment s is
    expert seg_expert[s]), as the grouped matmul takes them."""

    def __init__(self, topk_ids, n_experts):
        self.topk = np.asarray(topk_ids)
        offs, self.row_index = group(self.topk, n_experts)
        active = np.nonzero(np.diff(offs))[0]
        self.seg_expert = active.astype(np.int32)
        self.seg_offsets = np.concatenate([offs[active], [offs[-1]]]).astype(np.int32)

    @property
    def n_seg(self) -> int:
        return int(self.seg_expert.shape[0])

    @property
    def m_total(self) -> int:
        return int(self.row_index.shape[0])

    @property
    def max_seg_rows(self) -> int:
        return int(np.diff(self.seg_offsets).max()) if self.n_seg else 0


def route(x_bits, r_bits, bias, k=16):
    """Top-k routing of every token, grouped by expert (compact segments)."""
    scores, _ = route_scores(x_bits, r_bits, bias)
    return Routing(topk(scores, k), np.asarray(r_bits).shape[0])


# ---------------------------------------------------------------------------
# Expert FFN after the gate_up matmul: SwiGLU, then the weighted combine
# ---------------------------------------------------------------------------

def silu(v):
    """SiLU: v·σ(v) = v / (1 + e^(−v)), fp64.  The activation of the per-expert
    SwiGLU ("Colibri Kimi K3 Metal 后端实现全解析", the silu_mul operation of the
    Metal API table and Phase 6's per-expert activation)."""
    v = np.asarray(v, np.float64)
    with np.errstate(over="ignore"):
        return v / (1.0 + np.exp(-v))


def swiglu(y, n_inter):
    """h[r, j] = silu(g[r, j])·u[r, j] with g = y[:, :n_inter] (the gate) and
    u = y[:, n_inter:2·n_inter] (the up projection) of a gate_up output y."""
    y = np.asarray(y, np.float64)
    return silu(y[:, :n_inter]) * y[:, n_inter:2 * n_inter]


SILU_SLOPE_MAX = 1.1   # bound on |d silu / dv| over the reals (the maximum is 1.09984 at v ≈ 2.40)


def swiglu_tolerance(y, tol_y, n_inter):
    """Bound on |h_gpu − h| before the output rounding when each gate and up
    value the GPU used is within tol_y of the exact one: silu moves by at most
    SILU_SLOPE_MAX·tol_g, so |Δh| <= SILU_SLOPE_MAX·tol_g·(|u| + tol_u) +
    |silu(g)|·tol_u, plus 1e-6·|h| + 1e-30 for the fp32 evaluation of silu·u."""
    y = np.asarray(y, np.float64)
    tol_y = np.broadcast_to(np.asarray(tol_y, np.float64), y.shape)
    g, u = y[:, :n_inter], y[:, n_inter:2 * n_inter]
    tg, tu = tol_y[:, :n_inter], tol_y[:, n_inter:2 * n_inter]
    h = silu(g) * u
    return SILU_SLOPE_MAX * tg * (np.abs(u) + tu) + np.abs(silu(g)) * tu + 1e-6 * np.abs(h) + 1e-30


def combine(o, topk_ids, weights_src, seg_offsets, row_index):
    """Weighted scatter-add of the expert outputs back to the tokens
    ("Colibri Kimi K3 Metal 后端实现全解析", Phase 6: output accumulation by
    weighted scatter-add into token space).  For token t and its slot j
    (expert e = topk[t, j]): w[t, j] = weights_src[t, e] / Σ_j' weights_src[t,
    topk[t, j']] -- the chosen experts' sigmoid weights renormalised to sum to
    one ("Kimi K3 迁移到 Google TPU 的可行性评估（v2）", §2: sigmoid + renormalize)
    -- and out[t] = Σ_j w[t, j]·o[r(t, j)], where r(t, j) is the row of token t
    in expert e's segment of the grouped order.  Returns (out, A) with
    A[t, c] = Σ_j |w[t, j]·o[r(t, j), c]|, fp64."""
    o = np.asarray(o, np.float64)
    topk_ids = np.asarray(topk_ids, np.int64)
    src = np.asarray(weights_src, np.float64)
    t, k = topk_ids.shape
    where = {}
    for e in range(len(seg_offsets) - 1):
        for r in range(int(seg_offsets[e]), int(seg_offsets[e + 1])):
            where[(e, int(row_index[r]))] = r
    out = np.zeros((t, o.shape[1]))
    a = np.zeros((t, o.shape[1]))
    for i in range(t):
        sel = src[i, topk_ids[i]]
        w = sel / sel.sum()
        for j in range(k):
            term = w[j] * o[where[(int(topk_ids[i, j]), i)]]
            out[i] += term
            a[i] += np.abs(term)
    return out, a


def route_score_bound(a, d):
    """Acceptance bound on a routing weight sigmoid(logit) evaluated in fp32
    rather than fp64, for logits accumulated as the GPU router accumulates
    them: the products x·r of two bf16 values are exact in fp32; they are
    summed in blocks of 32 (a tree of at most 5 roundings plus the add into
    the running sum), the blocks of a token-expert pair accumulate in eight
    interleaved chains of at most d/32 steps in all, and the eight chain sums
    are added in sequence (7 roundings).  With u = 2^-24 the logit's error is
    then at most n·u·A, n = d/32 + 12, A = Σ|x·r| (the second output of
    route_scores), and the bound doubles it for margin.  The sigmoid's slope is
    at most 1/4, and its own fp32 evaluation plus the fp32 add of the bias cost
    a few ulps of 1, covered by 1e-6.  The pages fix no precision for the
    router (its scores only choose experts and weigh their outputs), so this is
    the reading used to accept an fp32 router; check_topk takes it as delta."""
    gamma = 2.0 * (np.asarray(d, np.float64) / 32.0 + 12.0) * 2.0 ** -24
    return 0.25 * gamma * np.asarray(a, np.float64) + 1e-6


def check_topk(topk_ids, scores, delta) -> dict:
    """Is a computed top-k a correct top-k for scores known only within
    ±delta?  Each row must hold k distinct experts, and every chosen expert e
    and unchosen f must satisfy score[e] + delta[e] + delta[f] >= score[f]
    (some scores within the error bounds rank e above f); consecutive picks
    must be in non-increasing order within the same margin.  Where the k-th
    and (k+1)-th scores are further apart than the margins, this leaves
    exactly the fp64 choice.  `delta` is per element, shaped like `scores`."""
    topk_ids = np.asarray(topk_ids, np.int64)
    scores = np.asarray(scores, np.float64)
    delta = np.broadcast_to(np.asarray(delta, np.float64), scores.shape)
    t, k = topk_ids.shape
    bad_rows = []
    for i in range(t):
        ids = topk_ids[i]
        if len(set(ids.tolist())) != k or ids.min() < 0 or ids.max() >= scores.shape[1]:
            bad_rows.append(i)
            continue
        chosen = np.zeros(scores.shape[1], bool)
        chosen[ids] = True
        lo_chosen = np.min(scores[i, ids] + delta[i, ids])
        hi_other = np.max(scores[i, ~chosen] - delta[i, ~chosen]) if (~chosen).any() else -np.inf
        ordered = np.all(scores[i, ids[:-1]] + delta[i, ids[:-1]] + delta[i, ids[1:]] >= scores[i, ids[1:]])
        if lo_chosen < hi_other or not ordered:
            bad_rows.append(i)
    ref = topk(scores, k)
    exact = int(np.sum(np.all(np.sort(ref, 1) == np.sort(topk_ids, 1), axis=1)))
    return dict(ok=not bad_rows, bad_rows=bad_rows[:10], n_bad=len(bad_rows),
                rows_equal_to_fp64_choice=exact, rows=t)


# ---------------------------------------------------------------------------
# Acceptance
# ---------------------------------------------------------------------------

REL_TOL = 2e-3
ABS_TOL = 1e-5


def check(y_bits, y_ref, a_ref, rel=REL_TOL, abs_=ABS_TOL) -> dict:
    """Per-element acceptance of a stored bf16 output.

    The computed value must lie within tol = rel·A + abs_ of the exact result
    y, and the output is that value rounded to bf16: so y_gpu passes iff it is
    one of the bf16 numbers between RNE(y - tol) and RNE(y + tol).  (Rounding
    to nearest is monotone, so that set is exactly {RNE(v) : |v - y| <= tol}.)
    The final rounding alone can move an output by up to 2**-8·|y|, more than
    2e-3·A when every product has the same sign, which is why it is allowed on
    top of the tolerance rather than inside it.

    Reports the raw max(|err|/tol), max |err| and the mean absolute error (the
    per-op maxAbs/MAE report of Colibri Kimi K3 Metal 后端实现全解析, Phase 5)."""
    y = bf16_to_f64(y_bits).reshape(np.shape(y_ref))
    y_ref = np.asarray(y_ref, np.float64)
    tol = rel * np.asarray(a_ref, np.float64) + abs_
    lo = round_to_bf16(y_ref - tol)
    hi = round_to_bf16(y_ref + tol)
    err = np.abs(y - y_ref)
    bad = ~((y >= lo) & (y <= hi))          # NaN in y counts as a failure
    return dict(ok=not bool(bad.any()), n_fail=int(bad.sum()), n=int(err.size),
                max_ratio=float(np.nanmax(err / tol)) if err.size else 0.0,
                max_abs=float(np.nanmax(err)) if err.size else 0.0,
                mae=float(np.nanmean(err)) if err.size else 0.0)
