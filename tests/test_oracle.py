"""Pins of the CPU oracle against what the pages and mathematics fix (CPU only).

Each pin is independent of the oracle's own code: golden values printed on the
pages (tests/golden/, each with its citation), exact rational brute force in
pure Python on tiny shapes, integer-exact cases, one-hot columns, row sums and
the tolerance checker's self-test.  `test_planted_mistakes` plants plausible
mistakes in the oracle (on the CPU) and checks that some pin catches each.
"""
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

RNG_SEED = 20261202


# --- independent exact helpers (pure Python, no numpy views, no oracle code) ---

def bf16_exact(bits: int) -> Fraction:
    return Fraction(struct.unpack(">f", struct.pack(">I", (int(bits) & 0xFFFF) << 16))[0])


def row_nibbles_le(words_row) -> list:
    """Codes of one row, read from the little-endian bytes of its uint32 words:
    code k lives in byte k // 2, low nibble when k is even."""
    raw = b"".join(struct.pack("<I", int(w)) for w in words_row)
    out = []
    for byte in raw:
        out.append(byte & 0xF)
        out.append(byte >> 4)
    return out


def brute_w_affine(codes, scale, bias):
    """Exact dequantised rows over the rationals."""
    out = []
    for j in range(codes.shape[0]):
        q = row_nibbles_le(codes[j])
        out.append([bf16_exact(scale[j][k // 64]) * q[k] + bf16_exact(bias[j][k // 64])
                    for k in range(len(q))])
    return out


def brute_affine(x_bits, codes, scale, bias):
    """Exact Y and A over the rationals."""
    t_, d = x_bits.shape
    n = codes.shape[0]
    y = [[Fraction(0)] * n for _ in range(t_)]
    a = [[Fraction(0)] * n for _ in range(t_)]
    wall = brute_w_affine(codes, scale, bias)
    for j in range(n):
        w = wall[j]
        for i in range(t_):
            for k in range(d):
                p = bf16_exact(x_bits[i][k]) * w[k]
                y[i][j] += p
                a[i][j] += abs(p)
    return y, a


def brute_mxfp4(x_bits, codes, e8m0, table):
    t_, d = x_bits.shape
    n = codes.shape[0]
    y = [[Fraction(0)] * n for _ in range(t_)]
    a = [[Fraction(0)] * n for _ in range(t_)]
    for j in range(n):
        c = []
        for byte in bytes(codes[j].tolist()):
            c += [byte & 0xF, byte >> 4]
        w = [Fraction(table[c[k]]) * Fraction(2) ** (int(e8m0[j][k // 32]) - 127) for k in range(d)]
        for i in range(t_):
            for k in range(d):
                p = bf16_exact(x_bits[i][k]) * w[k]
                y[i][j] += p
                a[i][j] += abs(p)
    return y, a


def rand_affine(rng, n, d):
    codes = rng.integers(0, 2 ** 32, size=(n, d // 8), dtype=np.uint64).astype(np.uint32)
    scale = synth.bf16_bits(rng.uniform(0.01, 0.05, size=(n, d // 64)))
    bias = synth.bf16_bits(rng.uniform(-0.4, 0.0, size=(n, d // 64)))
    return codes, scale, bias


def rand_x(rng, t, d):
    return synth.bf16_bits(rng.standard_normal((t, d)))


# --- pins ------------------------------------------------------------------

def pin_worked_example(golden):
    g = golden("affine_worked_example.json")
    q = list(g["q"]) + [0] * (64 - len(g["q"]))
    word = [sum(q[8 * i + j] << (4 * j) for j in range(8)) for i in range(8)]
    codes = np.array([word], np.uint32)
    scale = synth.bf16_bits(np.array([[g["scale"]]]))
    bias = synth.bf16_bits(np.array([[g["bias"]]]))
    w = oracle.dequant_affine(codes, scale, bias)
    assert w[0, :4].tolist() == g["w"], w[0, :4]
    # the same values reach the output through the contraction (one-hot rows of X)
    x = np.zeros((4, 64))
    x[np.arange(4), np.arange(4)] = 1.0
    y, _ = oracle.gemm_affine(synth.bf16_bits(x), codes, scale, bias)
    assert y[:, 0].tolist() == g["w"]


def pin_nibble_order(golden):
    g = golden("nibble_order.json")
    assert oracle.affine_codes(np.array([g["affine_words"]], np.uint32))[0].tolist() == g["affine_codes"]
    assert oracle.mxfp4_codes(np.array([g["mxfp4_bytes"]], np.uint8))[0].tolist() == g["mxfp4_codes"]


def pin_e2m1(golden):
    g = golden("e2m1_ocp_mx.json")
    v = oracle.e2m1_value(np.arange(16))
    assert v.tolist() == g["values_by_code"]
    assert np.signbit(v[8]) and not np.signbit(v[0])
    e = oracle.e8m0_value(np.array(g["e8m0"]["E"]))
    assert e.tolist() == [2.0 ** p for p in g["e8m0"]["log2_scale"]]
    assert np.isnan(oracle.e8m0_value(255))


def pin_brute_affine(shapes=((1, 1, 64), (2, 2, 128), (3, 7, 192), (5, 33, 64))):
    rng = np.random.default_rng(RNG_SEED)
    for t, n, d in shapes:
        codes, scale, bias = rand_affine(rng, n, d)
        x = rand_x(rng, t, d)
        y, a = oracle.gemm_affine(x, codes, scale, bias)
        ye, ae = brute_affine(x, codes, scale, bias)
        for i in range(t):
            for j in range(n):
                assert abs(y[i, j] - float(ye[i][j])) <= 1e-12 * float(ae[i][j]) + 1e-300, (t, n, d, i, j)
                assert abs(a[i, j] - float(ae[i][j])) <= 1e-12 * float(ae[i][j])


def pin_brute_mxfp4(golden, shapes=((1, 1, 32), (2, 2, 64), (3, 7, 96), (5, 33, 32))):
    table = golden("e2m1_ocp_mx.json")["values_by_code"]
    rng = np.random.default_rng(RNG_SEED + 1)
    for t, n, d in shapes:
        codes = rng.integers(0, 256, size=(n, d // 2)).astype(np.uint8)
        e8m0 = rng.integers(100, 140, size=(n, d // 32)).astype(np.uint8)
        x = rand_x(rng, t, d)
        y, a = oracle.gemm_mxfp4(x, codes, e8m0)
        ye, ae = brute_mxfp4(x, codes, e8m0, table)
        for i in range(t):
            for j in range(n):
                assert abs(y[i, j] - float(ye[i][j])) <= 1e-12 * float(ae[i][j]) + 1e-300, (t, n, d, i, j)
                assert abs(a[i, j] - float(ae[i][j])) <= 1e-12 * float(ae[i][j])


def pin_integer_exact():
    """scale 1, bias 0 and integer x: every result is an exact integer."""
    rng = np.random.default_rng(RNG_SEED + 2)
    n, d, t = 9, 192, 3
    codes = rng.integers(0, 2 ** 32, size=(n, d // 8), dtype=np.uint64).astype(np.uint32)
    one = synth.bf16_bits(np.ones((n, d // 64)))
    zero = synth.bf16_bits(np.zeros((n, d // 64)))
    xi = rng.integers(-3, 4, size=(t, d))
    y, _ = oracle.gemm_affine(synth.bf16_bits(xi.astype(float)), codes, one, zero)
    q = np.array([row_nibbles_le(codes[j]) for j in range(n)])
    assert np.array_equal(y, (xi @ q.T).astype(float))


def pin_one_hot_and_row_sums():
    rng = np.random.default_rng(RNG_SEED + 3)
    n, d = 5, 128
    codes, scale, bias = rand_affine(rng, n, d)
    wref = brute_w_affine(codes, scale, bias)
    y, _ = oracle.gemm_affine(synth.bf16_bits(np.eye(d)), codes, scale, bias)
    # one-hot row k of X returns column k of Ŵ, i.e. y[k, j] = ŵ[j, k], exactly
    assert np.array_equal(y, np.array([[float(wref[j][k]) for j in range(n)] for k in range(d)]))
    ys, _ = oracle.gemm_affine(synth.bf16_bits(np.ones((1, d))), codes, scale, bias)
    ye, _ = brute_affine(synth.bf16_bits(np.ones((1, d))), codes, scale, bias)
    for j in range(n):
        assert abs(ys[0, j] - float(ye[0][j])) <= 1e-12 * abs(float(ye[0][j])) + 1e-300


def pin_checker():
    rng = np.random.default_rng(RNG_SEED + 4)
    y = rng.standard_normal(50)
    a = 10.0 * np.abs(y) + 10.0              # tolerance well above one bf16 ulp of y
    bits = synth.bf16_bits(y)
    yb = oracle.bf16_to_f64(bits)
    assert oracle.check(bits, yb, a)["ok"]
    bad = yb.copy()
    bad[7] += 1.5 * (2e-3 * a[7] + 1e-5)
    assert not oracle.check(synth.bf16_bits(bad), yb, a)["ok"]
    nan = bits.copy()
    nan[3] = 0x7FC0
    assert not oracle.check(nan, yb, a)["ok"]
    # the correctly rounded output of an exact value whose products all share a
    # sign passes even though its rounding error exceeds 2e-3·A; one bf16 step
    # further does not
    y_ex, a_ex = 2.054577350616455, 2.785332202911377
    assert oracle.check(np.array([0x4003], np.uint16), np.array([y_ex]), np.array([a_ex]))["ok"]   # 2.046875
    assert not oracle.check(np.array([0x4002], np.uint16), np.array([y_ex]), np.array([a_ex]))["ok"]  # 2.03125
    assert oracle.check(np.array([0x4004], np.uint16), np.array([y_ex]), np.array([a_ex]))["ok"]   # 2.0625


def pin_router_hand_worked():
    """Scores and selections worked by hand.  Token 0 reads feature 0, token 1
    feature 1; R's rows give logits (2, 0, -1, 2, 0) and (0, 2, -1, 2, 0), and
    the bias (0, 0, 0, -1/4, 1/2) lifts expert 4 to sigmoid(0) + 1/2 = 1 and
    pushes expert 3 to sigmoid(2) - 1/4 < sigmoid(2) but > 1/2."""
    d = 8
    x = np.zeros((2, d))
    x[0, 0] = 1.0
    x[1, 1] = 1.0
    r = np.zeros((5, d))
    r[0, 0] = 2.0
    r[1, 1] = 2.0
    r[2, :2] = -1.0
    r[3, :2] = 2.0
    bias = np.array([0.0, 0.0, 0.0, -0.25, 0.5], np.float32)
    scores, a = oracle.route_scores(synth.bf16_bits(x), synth.bf16_bits(r), bias)
    assert scores[0, 1] == 0.5 and scores[1, 0] == 0.5          # sigmoid(0) exactly
    assert scores[0, 4] == 1.0 and scores[1, 4] == 1.0          # sigmoid(0) + 1/2
    assert scores[0, 2] < 0.5 and scores[0, 0] > scores[0, 3] > 0.5
    assert a[0, 3] == 2.0 and a[1, 2] == 1.0                      # Σ|x·r|
    assert oracle.topk(scores, 3).tolist() == [[4, 0, 3], [4, 1, 3]]
    # equal scores go to the lower expert id, in the choice and in the order
    tie = np.array([[0.3, 0.7, 0.7, 0.1, 0.7]])
    assert oracle.topk(tie, 2).tolist() == [[1, 2]]
    assert oracle.topk(tie, 4).tolist() == [[1, 2, 4, 0]]


def pin_router_full_sort():
    """The vectorised routing against a naive per-token full sort in Python floats."""
    import math
    x, r, bias = synth.router_inputs(1004, t=24, d=256, experts=48)
    rt = oracle.route(x, r, bias, k=8)
    xf = [[float(v) for v in row] for row in oracle.bf16_to_f64(x)]
    rf = [[float(v) for v in row] for row in oracle.bf16_to_f64(r)]
    for tok in range(24):
        sc = []
        for e in range(48):
            lg = math.fsum(xf[tok][j] * rf[e][j] for j in range(256))
            sc.append((1.0 / (1.0 + math.exp(-lg)) + float(bias[e]), e))
        sc.sort(key=lambda p: (-p[0], p[1]))
        assert [e for _, e in sc[:8]] == rt.topk[tok].tolist()


def pin_topk_non_finite():
    """Worked row: 2.0 first; the two 0.5 by id; -0 and +0 equal, by id; then
    -1.0; -inf after every finite score; NaN last, by id."""
    nan, inf = float("nan"), float("inf")
    row = np.array([[0.5, -inf, nan, 0.5, -0.0, 0.0, -inf, 2.0, nan, -1.0]])
    assert oracle.topk(row, 10)[0].tolist() == [7, 0, 3, 4, 5, 9, 1, 6, 2, 8]
    assert oracle.topk(row, 3)[0].tolist() == [7, 0, 3]


def pin_silu():
    """SiLU written out: σ(1) = 1/(1 + e^−1) = 0.7310585786300049, so
    silu(1) = 0.7310585786300049 and silu(−1) = −0.2689414213699951; silu(0) = 0;
    silu(v) − silu(−v) = v for every v; silu(v) -> v for large v."""
    assert oracle.silu(0.0) == 0.0
    assert abs(oracle.silu(1.0) - 0.7310585786300049) <= 1e-15
    assert abs(oracle.silu(-1.0) + 0.2689414213699951) <= 1e-15
    v = np.linspace(-30.0, 30.0, 121)
    assert np.max(np.abs(oracle.silu(v) - oracle.silu(-v) - v)) <= 1e-13
    assert abs(oracle.silu(40.0) - 40.0) <= 1e-12 and abs(oracle.silu(-40.0)) <= 1e-15
    # the slope bound the SwiGLU tolerance uses holds on a fine grid
    grid = np.linspace(-20.0, 20.0, 400001)
    assert np.max(np.abs(np.diff(oracle.silu(grid)) / np.diff(grid))) <= oracle.SILU_SLOPE_MAX


def pin_swiglu_tolerance():
    """The SwiGLU acceptance bound, hand-worked on two elements: g = 0, u = 1
    with both tolerances 1e-3 gives 1.1·1e-3·(1 + 1e-3) = 1.1011e-3 (silu(0) and
    h are 0); g = 2, u = −3 with tol_g = 0.01, tol_u = 0.02 gives
    1.1·0.01·3.02 + silu(2)·0.02 + 1e-6·|silu(2)·(−3)| = 0.06845716790158315
    (silu(2) = 2/(1 + e^−2) = 1.7615941559557646).  And it is a bound: at
    every corner g ± tol_g, u ± tol_u of a grid of values, the exact SwiGLU
    moves by no more than it."""
    y = np.array([[0.0, 2.0, 1.0, -3.0]])
    tol = np.array([[1e-3, 1e-2, 1e-3, 2e-2]])
    b = oracle.swiglu_tolerance(y, tol, 2)
    assert abs(b[0, 0] - 1.1011e-3) <= 1e-15 and abs(b[0, 1] - 0.06845716790158315) <= 1e-15
    g = np.linspace(-12.0, 12.0, 97)
    u = np.linspace(-5.0, 5.0, 41)
    gg, uu = [a.reshape(1, -1) for a in np.meshgrid(g, u)]
    for rel in (1e-3, 0.05, 0.5):
        tg, tu = rel * (np.abs(gg) + 0.1), rel * (np.abs(uu) + 0.2)
        bound = oracle.swiglu_tolerance(np.concatenate([gg, uu], axis=1),
                                        np.concatenate([tg, tu], axis=1), gg.shape[1])
        h = gg / (1.0 + np.exp(-gg)) * uu
        for sg in (-1.0, 1.0):
            for su in (-1.0, 1.0):
                g2, u2 = gg + sg * tg, uu + su * tu
                assert np.all(np.abs(g2 / (1.0 + np.exp(-g2)) * u2 - h) <= bound)


def sim_router_logit_f32(xv, rv):
    """One logit summed in fp32 the way the GPU router sums it: products exact
    (bf16 x bf16), 32-product blocks as a pairwise tree, block sums added into
    eight chains (chain w takes 64-code pieces w, w + 8, ...), the chain sums
    then added in order."""
    p = (xv.astype(np.float32) * rv.astype(np.float32)).astype(np.float32)
    d = p.shape[0]
    chains = [np.float32(0.0)] * 8
    for piece in range((d + 63) // 64):
        for half in range(2):
            blk = np.zeros(32, np.float32)
            seg = p[64 * piece + 32 * half:64 * piece + 32 * half + 32]
            blk[:seg.shape[0]] = seg
            while blk.shape[0] > 1:
                blk = (blk[0::2] + blk[1::2]).astype(np.float32)
            chains[piece % 8] = np.float32(chains[piece % 8] + blk[0])
    total = np.float32(0.0)
    for c in chains:
        total = np.float32(total + c)
    return total


def pin_route_score_bound():
    """The router's score bound, hand-worked: A = 1, d = 64 gives
    0.25·2·(2 + 12)·2^-24 + 1e-6 = 1.4172325134277343e-06; A = 10, d = 3584
    gives 0.25·2·124·2^-24·10 + 1e-6 = 3.7954879760742185e-05.  And it bounds
    an fp32 evaluation in the GPU's summation order: every simulated sigmoid
    score, same-sign and mixed-sign inputs, lies within it of the fp64 one; a
    score moved by twice the bound is rejected."""
    assert abs(oracle.route_score_bound(1.0, 64) - 1.4172325134277343e-06) <= 1e-21
    assert abs(oracle.route_score_bound(10.0, 3584) - 3.7954879760742185e-05) <= 1e-19
    rng = np.random.default_rng(RNG_SEED + 31)
    for d in (64, 96, 1024, 3584):
        for trial in range(6):
            if trial % 2:
                xv = oracle.bf16_to_f64(synth.bf16_bits(rng.uniform(0.5, 2.0, d)))
                rv = oracle.bf16_to_f64(synth.bf16_bits(rng.uniform(0.001, 0.02, d)))
            else:
                xv = oracle.bf16_to_f64(synth.bf16_bits(rng.standard_normal(d)))
                rv = oracle.bf16_to_f64(synth.bf16_bits(rng.normal(0.0, 0.02, d)))
            logit64 = float(np.dot(xv, rv))
            a = float(np.dot(np.abs(xv), np.abs(rv)))
            l32 = sim_router_logit_f32(xv, rv)
            s32 = float(np.float32(1.0) / (np.float32(1.0) + np.exp(-l32, dtype=np.float32)))
            s64 = 1.0 / (1.0 + np.exp(-logit64))
            bound = float(oracle.route_score_bound(a, d))
            assert abs(s32 - s64) <= bound, (d, trial, abs(s32 - s64), bound)
            assert not abs((s64 + 2.0 * bound) - s64) <= bound


def pin_swiglu_literal():
    """Gate first, up second: y = [1, −1 | 2, 3] -> [silu(1)·2, silu(−1)·3]."""
    h = oracle.swiglu(np.array([[1.0, -1.0, 2.0, 3.0]]), 2)
    assert np.allclose(h, [[1.4621171572600098, -0.8068242641099853]], rtol=0, atol=1e-15)


def pin_combine_hand_worked():
    """Two tokens, top-2 of three experts.  Token 0 picks experts 2 (weight 0.6)
    and 0 (0.2): renormalised 0.75 and 0.25; token 1 picks 0 (0.5) and 1 (0.25):
    2/3 and 1/3.  Grouped rows: expert 0 -> tokens 0, 1 (rows 0, 1), expert 1 ->
    token 1 (row 2), expert 2 -> token 0 (row 3)."""
    topk_ids = np.array([[2, 0], [0, 1]])
    src = np.array([[0.2, 0.9, 0.6], [0.5, 0.25, 0.1]])
    offs, rows = oracle.group(topk_ids, 3)
    assert offs.tolist() == [0, 2, 3, 4] and rows.tolist() == [0, 1, 1, 0]
    o = np.array([[1.0, 2.0], [3.0, 4.0], [5.0, 6.0], [7.0, 8.0]])
    out, a = oracle.combine(o, topk_ids, src, offs, rows)
    assert np.allclose(out, [[5.5, 6.5], [11.0 / 3.0, 14.0 / 3.0]], rtol=0, atol=1e-14)
    assert np.allclose(a, out, rtol=0, atol=1e-14)   # all terms positive


def pin_quantize_int8():
    """absmax 127 gives s = 1 exactly, so x_q = round-half-even(x): 2.5 -> 2,
    -2.5 -> -2, 100.5 -> 100, 101.5 -> 102, 0.375 -> 0; absmax 254 halves
    everything; an all-zero row quantises to zeros with s = 0."""
    vals = np.array([[127.0, -3.0, 2.5, -2.5, 0.375, 100.5, 101.5]])
    q, s = oracle.quantize_rows_int8(oracle.f64_to_bf16_bits(vals))
    assert s.tolist() == [1.0] and q.tolist() == [[127, -3, 2, -2, 0, 100, 102]]
    q, s = oracle.quantize_rows_int8(oracle.f64_to_bf16_bits(np.array([[254.0, 5.0, -7.0, 3.0]])))
    assert s.tolist() == [2.0] and q.tolist() == [[127, 2, -4, 2]]   # 2.5 -> 2, -3.5 -> -4, 1.5 -> 2
    q, s = oracle.quantize_rows_int8(np.zeros((1, 64), np.uint16))
    assert s.tolist() == [0.0] and not q.any()


def pin_deferred_brute():
    """The deferred GEMV written out element by element from its definition on
    small shapes (Python ints and floats), y and the size of its terms A =
    s_x·Σ_g (|scale·isum| + |bias·xsum|), and the integer-exact case: scale
    1, bias 0 and integer x with absmax 127 make y = Σ x·q exactly."""
    rng = np.random.default_rng(RNG_SEED + 21)
    for n, d in ((3, 64), (5, 192)):
        w = rand_affine(rng, n, d)
        x = oracle.f64_to_bf16_bits(rng.standard_normal((1, d)))
        y, a = oracle.gemv_affine_deferred(x, *w)
        xf = [float(v) for v in oracle.bf16_to_f64(x)[0]]
        amax = np.float32(max(abs(v) for v in xf))
        sx = np.float32(amax / np.float32(127.0))
        xq = [int(np.rint(np.float32(np.float32(v) / sx))) for v in xf]
        codes = oracle.affine_codes(w[0])
        for r in range(n):
            total = 0.0
            for gi in range(d // 64):
                isum = sum(xq[k] * int(codes[r, k]) for k in range(64 * gi, 64 * gi + 64))
                xsum = sum(xq[64 * gi:64 * gi + 64])
                total += float(oracle.bf16_to_f64(w[1][r, gi])) * isum + float(oracle.bf16_to_f64(w[2][r, gi])) * xsum
            assert abs(float(sx) * total - y[r]) <= 1e-12 * max(a[r], 1e-30)
            size = 0.0
            for gi in range(d // 64):
                isum = sum(xq[k] * int(codes[r, k]) for k in range(64 * gi, 64 * gi + 64))
                xsum = sum(xq[64 * gi:64 * gi + 64])
                size += abs(float(oracle.bf16_to_f64(w[1][r, gi])) * isum) + abs(float(oracle.bf16_to_f64(w[2][r, gi])) * xsum)
            assert abs(float(sx) * size - a[r]) <= 1e-12 * float(sx) * size
    n, d = 4, 128
    codes = rng.integers(0, 2 ** 32, (n, d // 8), dtype=np.uint64).astype(np.uint32)
    ones = np.full((n, d // 64), 0x3F80, np.uint16)
    zeros = np.zeros((n, d // 64), np.uint16)
    xi = rng.integers(-127, 128, (1, d)).astype(np.float64)
    xi[0, 0] = 127.0
    y, _ = oracle.gemv_affine_deferred(oracle.f64_to_bf16_bits(xi), codes, ones, zeros)
    assert np.array_equal(y, (oracle.affine_codes(codes) * xi.astype(np.int64)).sum(axis=1).astype(np.float64))


def pin_group_literal():
    """Grouping written out by hand: token 0 picks experts (1, 0), token 1 (0, 3)."""
    offs, rows = oracle.group(np.array([[1, 0], [0, 3]]), 4)
    assert offs.tolist() == [0, 2, 3, 3, 4]         # expert 2 has an empty segment
    assert rows.tolist() == [0, 1, 0, 1]            # tokens ascend inside a segment
    rt = oracle.Routing(np.array([[1, 0], [0, 3]]), 4)
    assert rt.seg_expert.tolist() == [0, 1, 3] and rt.seg_offsets.tolist() == [0, 2, 3, 4]
    assert rt.max_seg_rows == 2 and rt.m_total == 4
    # invariants on a routed workload: every token once per chosen expert, segments full
    x, r, bias = synth.router_inputs(1005, t=40, d=128, experts=32)
    rt = oracle.route(x, r, bias, k=6)
    assert rt.m_total == 240 and rt.seg_offsets[-1] == 240
    seen = {}
    for s in range(rt.n_seg):
        rows = rt.row_index[rt.seg_offsets[s]:rt.seg_offsets[s + 1]]
        assert len(rows) > 0 and np.all(np.diff(rows) > 0)
        for t in rows:
            seen.setdefault(int(t), []).append(int(rt.seg_expert[s]))
    for t in range(40):
        assert sorted(seen[t]) == sorted(rt.topk[t].tolist())


def pin_check_topk():
    """The top-k acceptance: a clear gap leaves only the exact choice; scores
    within the margins may come in either order."""
    scores = np.array([[0.9, 0.5, 0.8, 0.1], [0.6, 0.60001, 0.2, 0.1]])
    delta = np.full(scores.shape, 1e-4)
    assert oracle.check_topk([[0, 2], [1, 0]], scores, delta)["ok"]
    assert oracle.check_topk([[0, 2], [0, 1]], scores, delta)["ok"]      # near tie, swapped
    assert not oracle.check_topk([[0, 1], [1, 0]], scores, delta)["ok"]  # 0.5 chosen over 0.8
    assert not oracle.check_topk([[2, 0], [1, 0]], scores, delta)["ok"]  # out of order
    assert not oracle.check_topk([[0, 0], [1, 0]], scores, delta)["ok"]  # repeated expert


def all_pins(golden):
    pin_worked_example(golden)
    pin_nibble_order(golden)
    pin_e2m1(golden)
    pin_brute_affine(shapes=((1, 3, 128), (2, 5, 192)))
    pin_brute_mxfp4(golden, shapes=((2, 3, 64), (1, 4, 96)))
    pin_integer_exact()
    pin_one_hot_and_row_sums()
    pin_checker()
    pin_router_hand_worked()
    pin_router_full_sort()
    pin_topk_non_finite()
    pin_group_literal()
    pin_check_topk()
    pin_silu()
    pin_swiglu_literal()
    pin_swiglu_tolerance()
    pin_route_score_bound()
    pin_combine_hand_worked()
    pin_quantize_int8()
    pin_deferred_brute()


# --- tests -----------------------------------------------------------------

def test_worked_example(golden):
    pin_worked_example(golden)


def test_nibble_order(golden):
    pin_nibble_order(golden)


def test_e2m1_and_e8m0(golden):
    pin_e2m1(golden)
    cfg = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0}
    vals = set(np.abs(oracle.e2m1_value(np.arange(16))).tolist())
    assert vals == cfg


def test_group_sizes(golden):
    g = golden("format_sizes.json")
    ga = g["affine_g64"]
    assert ga["code_bytes"] * 2 == ga["codes_per_group"]
    assert ga["code_bytes"] + ga["metadata_bytes"] == ga["group_bytes"]
    assert round(100 * ga["group_bytes"] / ga["bf16_bytes"], 1) == ga["fraction_of_bf16_percent"]
    w = synth.affine_weights(5, 7, 192)
    assert w.codes.nbytes + w.scale.nbytes + w.bias.nbytes == ga["group_bytes"] * 7 * 192 // 64
    m = synth.mxfp4_weights(5, 7, 96, synth.S_GU_CODES, synth.S_GU_E8M0, 0)
    assert (m.codes.nbytes + m.e8m0.nbytes) * 8 == g["mxfp4_g32"]["bits_per_weight"] * 7 * 96
    # decode workload: 13824 x 5120 affine weights pack to 39,813,120 bytes
    assert 13824 * 5120 // 64 * ga["group_bytes"] == 39_813_120


def test_bruteforce_affine():
    pin_brute_affine()


def test_bruteforce_mxfp4(golden):
    pin_brute_mxfp4(golden)


def test_integer_exact():
    pin_integer_exact()


def test_one_hot_and_row_sums():
    pin_one_hot_and_row_sums()


def test_checker():
    pin_checker()


def test_bf16_rounding_helper():
    vals = np.array([0.0, -0.0, 1.0, -3.0, 255.0, 256.0, 257.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8,
                     2.0 ** -130, 3.0e38, 1e39])
    got = oracle.f64_to_bf16_bits(vals)
    # hand-derived patterns: 257 ties to 256; 1+2^-8 ties to 1; 1+3*2^-8 ties up to 1+2^-6;
    # 2^-130 is the subnormal 8 * 2^-133; 1e39 overflows to inf
    exp = [0x0000, 0x8000, 0x3F80, 0xC040, 0x437F, 0x4380, 0x4380, 0x3F80, 0x3F82, 0x0008, 0x7F62, 0x7F80]
    assert got.tolist() == exp


def test_round_to_bf16_matches_scalar_rounding():
    rng = np.random.default_rng(RNG_SEED + 6)
    v = np.concatenate([rng.standard_normal(2000) * 10.0 ** rng.integers(-40, 39, 2000),
                        [0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 257.0, 2.0 ** -130,
                         3 * 2.0 ** -134, 3.0e38, 3.3961e38, 3.4e38, -1e39, 2.0 ** -126 - 2.0 ** -134]])
    bits = oracle.f64_to_bf16_bits(v)
    ref = oracle.bf16_to_f64(bits)
    got = oracle.round_to_bf16(v)
    assert np.array_equal(np.signbit(got), np.signbit(ref))
    assert np.array_equal(got, ref)


def test_router_hand_worked():
    pin_router_hand_worked()


def test_router_full_sort():
    pin_router_full_sort()


def test_topk_non_finite():
    pin_topk_non_finite()


def test_silu():
    pin_silu()


def test_swiglu_tolerance():
    pin_swiglu_tolerance()


def test_route_score_bound():
    pin_route_score_bound()


def test_swiglu_literal():
    pin_swiglu_literal()


def test_combine_hand_worked():
    pin_combine_hand_worked()


def test_quantize_int8():
    pin_quantize_int8()


def test_deferred_brute():
    pin_deferred_brute()


def test_group_literal():
    pin_group_literal()


def test_check_topk():
    pin_check_topk()


def test_grouped_and_sampled(golden):
    rng = np.random.default_rng(RNG_SEED + 5)
    e_count, n, d, t = 4, 6, 64, 5
    ws = {e: rand_affine(rng, n, d) for e in range(e_count)}
    x = rand_x(rng, t, d)
    seg_expert = np.array([0, 2, 3], np.int32)
    seg_offsets = np.array([0, 2, 2, 5], np.int32)     # includes an empty segment
    row_index = np.array([4, 1, 0, 3, 4], np.int32)
    y, a = oracle.grouped(x, row_index, seg_expert, seg_offsets,
                          lambda e: oracle.dequant_affine(*ws[e]))
    for s in range(3):
        for r in range(seg_offsets[s], seg_offsets[s + 1]):
            ye, ae = brute_affine(x[row_index[r]][None, :], *ws[seg_expert[s]])
            for j in range(n):
                assert abs(y[r, j] - float(ye[0][j])) <= 1e-12 * float(ae[0][j])
    pairs = [(0, 1), (4, 5), (2, 0)]
    ys, as_ = oracle.sampled(x, lambda j: oracle.dequant_affine(*ws[1])[j], pairs)
    yf, af = oracle.gemm_affine(x, *ws[1])
    for i, (tt, j) in enumerate(pairs):
        assert abs(ys[i] - yf[tt, j]) <= 1e-12 * af[tt, j]


def _quantize_half_away(x_bits):
    """A plausible mistake: ties rounded away from zero instead of to even."""
    x = oracle.bf16_to_f64(x_bits).astype(np.float32).reshape(-1, np.shape(x_bits)[-1])
    s = (np.max(np.abs(x), axis=1) / np.float32(127.0)).astype(np.float32)
    v = x / np.where(s > 0, s, np.float32(1.0))[:, None]
    q = np.trunc(v + np.float32(0.5) * np.sign(v))
    return np.where(s[:, None] > 0, q, 0).astype(np.int64), s


MUTATIONS = {
    "drop_bias": ("dequant_affine", lambda orig: (lambda c, s, b: orig(c, s, np.zeros_like(b)))),
    "nibbles_high_first": ("affine_codes", lambda orig: (lambda w: orig(w).reshape(-1, 8)[:, ::-1].reshape(orig(w).shape))),
    "group_index_mod": ("dequant_affine", lambda orig: (
        lambda c, s, b: oracle.affine_codes(c) * np.tile(oracle.bf16_to_f64(s), (1, 64))
        + np.tile(oracle.bf16_to_f64(b), (1, 64)))),
    "e8m0_bias_128": ("e8m0_value", lambda orig: (lambda e: orig(e) / 2.0)),
    "e2m1_no_subnormal": ("e2m1_value", lambda orig: (
        lambda c: np.where((np.asarray(c) & 7) == 1, np.sign(orig(c)) * 1.0, orig(c)))),
    "transposed_w": ("matmul", lambda orig: (
        lambda x, w: orig(x, np.asarray(w)[::-1]) if np.shape(w)[0] > 1 else orig(x, np.asarray(w) * 1.5))),
    "mxfp4_high_nibble_first": ("mxfp4_codes", lambda orig: (
        lambda b: orig(b).reshape(-1, 2)[:, ::-1].reshape(orig(b).shape))),
    "checker_too_loose": ("check", lambda orig: (lambda *a, **k: dict(orig(*a, **k), ok=True))),
    "checker_rounds_wrong_way": ("round_to_bf16", lambda orig: (lambda v: orig(v) * (1 + 2.0 ** -6))),
    "router_bias_ignored": ("route_scores", lambda orig: (lambda x, r, b: orig(x, r, None))),
    "router_sigmoid_negated": ("route_scores", lambda orig: (
        lambda x, r, b: (lambda sa: (1.0 - sa[0] + 2 * (0 if b is None else np.asarray(b, np.float64))[None, :], sa[1]))(orig(x, r, b)))),
    "topk_ties_to_higher_id": ("topk", lambda orig: (
        lambda s, k: np.lexsort((-np.broadcast_to(np.arange(np.shape(s)[1]), np.shape(s)), -np.asarray(s, np.float64)),
                                axis=1)[:, :k])),
    "topk_ascending": ("topk", lambda orig: (lambda s, k: orig(-np.asarray(s, np.float64), k))),
    "group_tokens_descending": ("group", lambda orig: (
        lambda tk, e: (lambda o: (o[0], np.concatenate([o[1][o[0][i]:o[0][i + 1]][::-1] for i in range(e)]).astype(np.int32)))(orig(tk, e)))),
    "check_topk_too_loose": ("check_topk", lambda orig: (lambda *a, **k: dict(orig(*a, **k), ok=True))),
    "silu_is_sigmoid": ("silu", lambda orig: (lambda v: 1.0 / (1.0 + np.exp(-np.asarray(v, np.float64))))),
    "silu_sign_flipped": ("silu", lambda orig: (lambda v: np.asarray(v, np.float64) / (1.0 + np.exp(np.asarray(v, np.float64))))),
    "swiglu_halves_swapped": ("swiglu", lambda orig: (
        lambda y, n: orig(np.concatenate([np.asarray(y)[:, n:2 * n], np.asarray(y)[:, :n]], axis=1), n))),
    "quantize_half_away": ("quantize_rows_int8", lambda orig: _quantize_half_away),
    "deferred_no_bias_correction": ("gemv_affine_deferred", lambda orig: (
        lambda x, c, s, b: orig(x, c, s, np.zeros_like(b)))),
    "swiglu_tolerance_10x_loose": ("swiglu_tolerance", lambda orig: (lambda y, t, n: 10.0 * orig(y, t, n))),
    "swiglu_tolerance_drops_up_term": ("swiglu_tolerance", lambda orig: (
        lambda y, t, n: orig(y, t, n) - np.abs(oracle.silu(np.asarray(y, np.float64)[:, :n]))
        * np.broadcast_to(np.asarray(t, np.float64), np.shape(y))[:, n:2 * n])),
    "deferred_size_drops_bias_term": ("gemv_affine_deferred", lambda orig: (
        lambda x, c, s, b: (orig(x, c, s, b)[0], orig(x, c, s, np.zeros_like(b))[1]))),
    "route_bound_10x_loose": ("route_score_bound", lambda orig: (lambda a, d: 10.0 * orig(a, d))),
    "route_bound_no_slope": ("route_score_bound", lambda orig: (lambda a, d: 4.0 * orig(a, d) - 3e-6)),
    "route_bound_100x_tight": ("route_score_bound", lambda orig: (lambda a, d: 0.01 * orig(a, d))),
    "combine_not_renormalised": ("combine", lambda orig: (
        lambda o, tk, src, so, ri: (lambda res, sums: (res[0] * sums, res[1] * sums))(
            orig(o, tk, src, so, ri),
            np.asarray(src, np.float64)[np.arange(np.shape(tk)[0])[:, None], np.asarray(tk)].sum(1)[:, None]))),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistakes(name, golden, monkeypatch):
    attr, make = MUTATIONS[name]
    monkeypatch.setattr(oracle, attr, make(getattr(oracle, attr)))
    with pytest.raises(AssertionError):
        all_pins(golden)
