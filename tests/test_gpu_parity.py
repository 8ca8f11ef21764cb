"""GPU parity: every libqmm kernel against the fp64 CPU oracle (needs an MI355X).

Acceptance per element: |y_gpu − y| ≤ 2e-3·Σ|x·ŵ| + 1e-5 with the bf16 output
widened exactly; integer-exact inputs must match bit for bit; outputs start as
a NaN sentinel so an unwritten element fails.  All inputs come from the seeded
generator; nothing expected is produced by the HIP path itself.
"""
import sys

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import bit_weight_quantized_amd as qmm  # noqa: E402

A, M = qmm.QMM_AFFINE4_G64, qmm.QMM_MXFP4_G32
NAN16 = 0x7FC0
DEV = "cuda"


def say(*a):
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qmm.load()
    yield
    torch.cuda.synchronize()


def dev(a, dtype=None):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    elif a.dtype == np.uint32:
        a = a.view(np.int32)
    return torch.from_numpy(a).to(DEV)


def host_u16(t):
    return t.cpu().numpy().view(np.uint16)


# Guard bands: every output buffer (and workspace, and packed blob) these tests
# hand to the library sits between 256 bytes and 4 KiB of canary bytes, which
# must be unchanged after the test -- a write before the start or past the end
# of an output fails the test even where it would not fault.
GUARD_LEAD, GUARD_TAIL, CANARY = 256, 4096, 0x5A
_guarded = []


def guarded(shape, fill, dtype):
    """A device tensor of `shape` filled with `fill`, carved out of a larger
    buffer whose guard bands hold CANARY bytes; checked after each test."""
    esize = torch.empty(0, dtype=dtype).element_size()
    n = int(np.prod(shape)) if len(shape) else 1
    lead, tail = GUARD_LEAD // esize, GUARD_TAIL // esize
    base = torch.empty(lead + n + tail, dtype=dtype, device=DEV)
    base.view(torch.uint8).fill_(CANARY)
    body = base[lead:lead + n]
    body.fill_(fill)
    _guarded.append((base, lead, n))
    return body.view(*shape)


@pytest.fixture(autouse=True)
def _check_guards():
    _guarded.clear()
    yield
    torch.cuda.synchronize()
    for base, lead, n in _guarded:
        raw = base.cpu().numpy().view(np.uint8)
        esize = raw.size // base.numel()
        before, after = raw[:lead * esize], raw[(lead + n) * esize:]
        assert np.all(before == CANARY) and np.all(after == CANARY), \
            f"bytes changed outside a {n}-element buffer: {np.count_nonzero(before != CANARY)} before, " \
            f"{np.count_nonzero(after != CANARY)} after"
    _guarded.clear()


def nan_out(*shape):
    return guarded(shape, NAN16, torch.int16)


def pack_affine(w):
    packed = guarded((qmm.qmm_packed_bytes(A, w.n, w.d),), 0, torch.uint8)
    qmm.qmm_pack(A, w.n, w.d, dev(w.codes), dev(w.scale), dev(w.bias), packed)
    return packed


def pack_mxfp4(w):
    packed = guarded((qmm.qmm_packed_bytes(M, w.n, w.d),), 0, torch.uint8)
    qmm.qmm_pack(M, w.n, w.d, dev(w.codes), dev(w.e8m0), None, packed)
    return packed


def rand_mxfp4(seed, n, d, e_lo=118, e_count=9):
    return synth.mxfp4_weights(seed, n, d, synth.S_GU_CODES, synth.S_GU_E8M0, 0, e_lo, e_count)


def assert_parity(y_bits, y_ref, a_ref, what):
    r = oracle.check(y_bits, y_ref, a_ref)
    say(what, {k: r[k] for k in ("n", "n_fail", "max_ratio", "max_abs")})
    assert r["ok"], (what, r)


# ---------------------------------------------------------------------------
# pack / unpack
# ---------------------------------------------------------------------------

def test_roundtrip_affine():
    say("roundtrip affine 37x192")
    w = synth.affine_weights(11, 37, 192)
    w.codes[0, :] = 0
    w.codes[1, :] = 0xFFFFFFFF
    p = pack_affine(w)
    c, s, b = (guarded(w.codes.shape, 0, torch.int32), guarded(w.scale.shape, 0, torch.int16),
               guarded(w.bias.shape, 0, torch.int16))
    qmm.qmm_unpack(A, w.n, w.d, p, c, s, b)
    torch.cuda.synchronize()
    assert np.array_equal(c.cpu().numpy().view(np.uint32), w.codes)
    assert np.array_equal(host_u16(s), w.scale) and np.array_equal(host_u16(b), w.bias)
    # header: the payload follows 256 header bytes and is 36 B per 64 weights
    assert p.numel() >= 256 + 37 * 192 * 36 // 64


def test_roundtrip_mxfp4_all_codes_and_scales():
    say("roundtrip mxfp4 33x96")
    w = rand_mxfp4(12, 33, 96)
    w.e8m0.reshape(-1)[:] = np.arange(w.e8m0.size) % 255        # every E8M0 in 0..254
    w.codes[0, :] = (np.arange(48) * 0x11 % 256).astype(np.uint8)
    p = pack_mxfp4(w)
    c, e = guarded(w.codes.shape, 0, torch.uint8), guarded(w.e8m0.shape, 0, torch.uint8)
    qmm.qmm_unpack(M, w.n, w.d, p, c, e, None)
    torch.cuda.synchronize()
    assert np.array_equal(c.cpu().numpy(), w.codes) and np.array_equal(e.cpu().numpy(), w.e8m0)


def test_pack_rejects_nan_scale_and_unpack_checks_header():
    say("pack NaN scale")
    w = rand_mxfp4(13, 8, 64)
    w.e8m0[3, 1] = 255
    with pytest.raises(qmm.QmmError) as ei:
        pack_mxfp4(w)
    assert ei.value.status == 8
    w2 = synth.affine_weights(14, 16, 128)
    p = pack_affine(w2)
    c = torch.empty(16 * 16, dtype=torch.int32, device=DEV)
    s = torch.empty(16 * 2, dtype=torch.int16, device=DEV)
    with pytest.raises(qmm.QmmError) as ei:
        qmm.qmm_unpack(A, 16, 64, p, c, s, s)                        # wrong d
    assert ei.value.status == 7
    with pytest.raises(qmm.QmmError) as ei:
        qmm.qmm_unpack(M, 16, 128, p, c, s, None)                    # wrong format
    assert ei.value.status == 7


def test_gpu_generator_matches_host():
    say("generator gpu vs host")
    import synth.gpu as sg
    t = torch.empty(1001, dtype=torch.uint8, device=DEV)
    sg.code_bytes(1003, synth.S_GU_CODES, 17, t, start_byte=13)
    assert np.array_equal(t.cpu().numpy(), synth.code_bytes(1003, synth.S_GU_CODES, 17, 1001, start_byte=13))
    e = torch.empty(777, dtype=torch.uint8, device=DEV)
    sg.small_int_u8(1003, synth.S_GU_E8M0, 17, e, 118, 9, start=5)
    assert np.array_equal(e.cpu().numpy(), synth.small_int(1003, synth.S_GU_E8M0, 17, 777, 118, 9, start=5))


# ---------------------------------------------------------------------------
# GEMV
# ---------------------------------------------------------------------------

def run_gemv(fmt, packed, w, x_bits):
    y = nan_out(w.n)
    if fmt == A:
        qmm.qmm_gemv(A, packed, w.n, w.d, dev(x_bits), y)
    else:
        qmm.qmm_gemv(M, packed, w.n, w.d, dev(x_bits), y)
    torch.cuda.synchronize()
    return host_u16(y)


@pytest.mark.parametrize("n,d", [(512, 256), (1, 64), (3, 64), (37, 192), (100, 576), (257, 1088),
                                 (1000, 5120), (5, 8704), (300, 65536)])
def test_gemv_affine(n, d):
    say("gemv affine", n, d)
    w = synth.affine_weights(1000 + n, n, d)
    x = synth.activations(2000 + d, synth.S_X, 1, d)
    y = run_gemv(A, pack_affine(w), w, x[0])
    yr, ar = oracle.gemm_affine(x, w.codes, w.scale, w.bias)
    assert_parity(y, yr[0], ar[0], f"gemv affine {n}x{d}")


def test_gemv_affine_decode_workload_full():
    """13824 x 5120, every output against the oracle."""
    say("gemv affine 13824x5120 full")
    cfg = synth.CONFIGS[1]
    w = synth.affine_weights(synth.seed_of(1), cfg["n"], cfg["d"])
    x = synth.activations(synth.seed_of(1), synth.S_X, 1, cfg["d"])
    y = run_gemv(A, pack_affine(w), w, x[0])
    yr, ar = oracle.gemm_affine(x, w.codes, w.scale, w.bias)
    assert_parity(y, yr[0], ar[0], "gemv affine 13824x5120")


@pytest.mark.parametrize("n,d,elo,ecount", [(1, 32, 118, 9), (7, 96, 118, 9), (100, 3584, 118, 9),
                                            (33, 3072, 118, 9), (64, 512, 1, 200), (9, 1056, 100, 60),
                                            (40, 20480, 118, 9)])
def test_gemv_mxfp4(n, d, elo, ecount):
    say("gemv mxfp4", n, d, elo, ecount)
    w = rand_mxfp4(3000 + n, n, d, elo, ecount)
    x = synth.activations(4000 + d, synth.S_X, 1, d)
    y = run_gemv(M, pack_mxfp4(w), w, x[0])
    yr, ar = oracle.gemm_mxfp4(x, w.codes, w.e8m0)
    # E8M0 up to 200 keeps every product and sum inside the fp32/bf16 range;
    # E8M0 = 1 exercises the smallest normal scale 2^-126
    assert_parity(y, yr[0], ar[0], f"gemv mxfp4 {n}x{d} E in [{elo}, {elo + ecount})")


@pytest.mark.parametrize("shapes,d", [((512, 128, 128), 512), ((300, 300), 1088), ((5120, 1024, 1024), 5120)])
def test_gemv_fused_projections(shapes, d):
    """Matrices that share one activation row -- a GQA Q/K/V triple, a gate/up
    pair ("LLM Decode / Prefill 优化案例（Metal）", Steps 8 and 9) -- run as one
    launch when packed as one matrix, their rows concatenated.  Each block of
    the fused output equals its own GEMV bit for bit (a row's result depends
    only on that row) and the oracle."""
    say("gemv fused projections", shapes, d)
    ws = [synth.affine_weights(5000 + i, n, d) for i, n in enumerate(shapes)]
    fused = synth.Affine(np.concatenate([w.codes for w in ws]), np.concatenate([w.scale for w in ws]),
                         np.concatenate([w.bias for w in ws]))
    x = synth.activations(5100 + d, synth.S_X, 1, d)
    yf = run_gemv(A, pack_affine(fused), fused, x[0])
    off = 0
    for i, w in enumerate(ws):
        ys = run_gemv(A, pack_affine(w), w, x[0])
        assert np.array_equal(yf[off:off + w.n], ys)
        yr, ar = oracle.gemm_affine(x, w.codes, w.scale, w.bias)
        assert_parity(yf[off:off + w.n], yr[0], ar[0], f"fused projection {i}: {w.n}x{d}")
        off += w.n


@pytest.mark.parametrize("fmt,small,d", [(A, 999, 5184), (A, 77, 2048), (M, 130, 3584), (A, 5, 8704),
                                         (M, 6, 20480)])
def test_gemv_split_quads_bitwise(fmt, small, d):
    """A matrix of few rows deals each quad's slabs to 2 or 4 waves and adds
    their per-slab partials in slab order; a matrix of more than 6144 rows
    keeps one wave per quad.  The first rows of a large matrix, packed as a
    matrix of their own, must give the same bits both ways (narrow last slab,
    several LDS passes, both formats), and meet the oracle."""
    big = 6400
    say("gemv split quads", fmt, small, big, d)
    if fmt == A:
        wb = synth.affine_weights(5300 + d, big, d)
        ws = synth.Affine(wb.codes[:small], wb.scale[:small], wb.bias[:small])
        pb, ps = pack_affine(wb), pack_affine(ws)
    else:
        wb = rand_mxfp4(5300 + d, big, d)
        ws = synth.MXFP4(wb.codes[:small], wb.e8m0[:small])
        pb, ps = pack_mxfp4(wb), pack_mxfp4(ws)
    x = synth.activations(5400 + d, synth.S_X, 1, d)
    yb = run_gemv(fmt, pb, wb, x[0])
    ysm = run_gemv(fmt, ps, ws, x[0])
    assert np.array_equal(yb[:small], ysm)
    if fmt == A:
        yr, ar = oracle.gemm_affine(x, ws.codes, ws.scale, ws.bias)
    else:
        yr, ar = oracle.gemm_mxfp4(x, ws.codes, ws.e8m0)
    assert_parity(ysm, yr[0], ar[0], f"gemv split quads {small}x{d}")


def run_gemv_int8(packed, n, d, x_bits):
    y = nan_out(n)
    qmm.qmm_gemv_int8(A, packed, n, d, dev(x_bits), y)
    torch.cuda.synchronize()
    return host_u16(y)


@pytest.mark.parametrize("n,d", [(512, 256), (37, 192), (300, 1088), (1000, 5120), (13824, 5120), (5, 57344)])
def test_gemv_int8(n, d):
    """The deferred-dequantisation GEMV against the oracle of the same method
    (int8 activations decided in fp32 on both sides, exact integer sums);
    its distance from the exact bf16 GEMV is reported, not asserted."""
    say("gemv int8", n, d)
    w = synth.affine_weights(6000 + n, n, d)
    x = synth.activations(6100 + d, synth.S_X, 1, d)
    y = run_gemv_int8(pack_affine(w), n, d, x[0])
    yr, ar = oracle.gemv_affine_deferred(x, w.codes, w.scale, w.bias)
    assert_parity(y, yr, ar, f"gemv int8 {n}x{d}")
    ye, ae = oracle.gemm_affine(x, w.codes, w.scale, w.bias)
    dev_exact = np.abs(oracle.bf16_to_f64(y) - ye[0]) / ae[0]
    say("gemv int8 vs exact", {"max_err_over_A": float(dev_exact.max()), "mean": float(dev_exact.mean())})


def test_gemv_int8_integer_exact_and_zero_row():
    """Scale 1, bias 0 and integer activations with absmax 127 make the
    quantisation the identity, so every sum is an exact integer below 2^24 in
    fp32 and the output is its one bf16 rounding, bit for bit; a zero row
    gives zeros."""
    say("gemv int8 integer exact")
    rng = np.random.default_rng(61)
    n, d = 64, 1088
    w = integer_affine(6200, n, d)
    xi = rng.integers(-8, 9, (1, d)).astype(np.float64)
    xi[0, 5] = 127.0
    x = oracle.f64_to_bf16_bits(xi)
    y = run_gemv_int8(pack_affine(w), n, d, x[0])
    exact = (oracle.affine_codes(w.codes) * xi.astype(np.int64)).sum(axis=1)
    assert np.all(np.abs(exact) < 2 ** 24)
    assert np.array_equal(oracle.bf16_to_f64(y), oracle.round_to_bf16(exact.astype(np.float64)))
    z = run_gemv_int8(pack_affine(w), n, d, np.zeros(d, np.uint16))
    assert not np.any(oracle.bf16_to_f64(z))


def integer_affine(seed, n, d):
    w = synth.affine_weights(seed, n, d)
    w.scale[:] = 0x3F80      # 1.0
    w.bias[:] = 0            # 0.0
    return w


def test_gemv_integer_exact():
    say("gemv integer exact")
    rng = np.random.default_rng(5)
    n, d = 300, 1088
    w = integer_affine(21, n, d)
    xi = rng.integers(-3, 4, size=(1, d)).astype(float)
    x = synth.bf16_bits(xi)
    yr, _ = oracle.gemm_affine(x, w.codes, w.scale, w.bias)
    # every partial sum is an integer below 2^24, exact in fp32, so both sides
    # round the same exact integer to bf16
    assert np.all(np.abs(yr) < 2 ** 24)
    y = run_gemv(A, pack_affine(w), w, x[0])
    assert np.array_equal(y, oracle.f64_to_bf16_bits(yr[0]))


# ---------------------------------------------------------------------------
# GEMM
# ---------------------------------------------------------------------------

def run_gemm(fmt, packed, n, d, x_bits):
    """qmm_gemm as a caller without a workspace of its own would call it:
    MXFP4 weights with none; affine weights (t >= 2) with the workspace they
    need (NaN-filled: its contents on entry must not matter)."""
    t = x_bits.shape[0]
    need = qmm.qmm_workspace_bytes(fmt, t, n, d) if fmt == A else 0
    ws = guarded((need // 4,), float("nan"), torch.float32) if need else None
    y = nan_out(t, n)
    qmm.qmm_gemm(fmt, packed, t, n, d, dev(x_bits), y, ws)
    torch.cuda.synchronize()
    return host_u16(y)


def run_gemm_tile(fmt, packed, n, d, x_bits):
    """qmm_gemm on the tile kernel (forced), with the workspace it asks for."""
    qmm.qmm_set_kernel(qmm.QMM_KERNEL_TILE)
    try:
        t = x_bits.shape[0]
        need = qmm.qmm_workspace_bytes(fmt, t, n, d)
        ws = guarded((need // 4,), float("nan"), torch.float32) if need else None
        y = nan_out(t, n)
        qmm.qmm_gemm(fmt, packed, t, n, d, dev(x_bits), y, ws)
        torch.cuda.synchronize()
    finally:
        qmm.qmm_set_kernel(qmm.QMM_KERNEL_AUTO)
    return host_u16(y)


@pytest.mark.parametrize("t,n,d", [(2, 5, 64), (3, 300, 320), (130, 257, 576), (129, 512, 1024),
                                   (300, 520, 640), (257, 256, 256), (513, 100, 5120),
                                   # d a multiple of 512 (whole-region weight descriptors), both
                                   # tile heights, n not a multiple of 4 or of 256, ragged t
                                   (200, 301, 512), (70, 259, 1024), (3, 1, 1536), (600, 517, 2048)])
def test_gemm_affine(t, n, d):
    say("gemm affine", t, n, d)
    w = synth.affine_weights(5000 + n, n, d)
    x = synth.activations(6000 + t, synth.S_X, t, d)
    y = run_gemm(A, pack_affine(w), n, d, x)
    yr, ar = oracle.gemm_affine(x, w.codes, w.scale, w.bias)
    assert_parity(y, yr, ar, f"gemm affine {t}x{n}x{d}")


@pytest.mark.parametrize("t,n,d,elo,ecount", [(2, 5, 32, 118, 9), (3, 300, 96, 118, 9),
                                              (130, 257, 3584, 118, 9), (257, 300, 3072, 118, 9),
                                              (64, 70, 1056, 100, 50), (33, 130, 2048, 118, 9),
                                              (300, 259, 1024, 100, 50)])
def test_gemm_mxfp4(t, n, d, elo, ecount):
    say("gemm mxfp4", t, n, d)
    w = rand_mxfp4(7000 + n, n, d, elo, ecount)
    x = synth.activations(8000 + t, synth.S_X, t, d)
    y = run_gemm(M, pack_mxfp4(w), n, d, x)
    yr, ar = oracle.gemm_mxfp4(x, w.codes, w.e8m0)
    assert_parity(y, yr, ar, f"gemm mxfp4 {t}x{n}x{d}")


@pytest.mark.parametrize("fmt,d", [(A, 512), (A, 576), (M, 512), (M, 1056)])
def test_gemm_256_row_tiles(fmt, d):
    """2048 x 4352 outputs: 272 tiles of 128 rows, more than a 256-CU chip has
    CUs, so the launcher takes the 256-row tile; d a multiple of 512 or not
    (whole-region or per-slab weight addressing), MXFP4 with a half K step."""
    t, n = 2048, 4352
    say("gemm 256-row tiles", fmt, t, n, d)
    x = synth.activations(6300 + d, synth.S_X, t, d)
    if fmt == A:
        w = synth.affine_weights(5300 + d, n, d)
        y = run_gemm(A, pack_affine(w), n, d, x)
        yr, ar = oracle.gemm_affine(x, w.codes, w.scale, w.bias)
    else:
        w = rand_mxfp4(7300 + d, n, d)
        y = run_gemm(M, pack_mxfp4(w), n, d, x)
        yr, ar = oracle.gemm_mxfp4(x, w.codes, w.e8m0)
    assert_parity(y, yr, ar, f"gemm 256-row tiles {fmt} {t}x{n}x{d}")


@pytest.mark.parametrize("fmt,t,n,d", [(A, 4, 130, 65536), (A, 70, 130, 65536), (A, 300, 97, 65536),
                                       (M, 4, 130, 65536), (M, 300, 97, 65504)])
def test_gemm_largest_d(fmt, t, n, d):
    """The largest reduction axis the layout takes (d = 65536, 128 slabs; and a
    narrow last slab for MXFP4): the few-row kernel, the tile kernel split along
    K and unsplit, both formats, against the oracle."""
    say("gemm largest d", fmt, t, n, d)
    x = synth.activations(6900 + t, synth.S_X, t, d)
    if fmt == A:
        w = synth.affine_weights(5900 + n, n, d)
        y = run_gemm(A, pack_affine(w), n, d, x)
        yr, ar = oracle.gemm_affine(x, w.codes, w.scale, w.bias)
    else:
        w = rand_mxfp4(7900 + n, n, d)
        need = qmm.qmm_workspace_bytes(M, t, n, d)
        ws = guarded((need // 4,), float("nan"), torch.float32) if need else None
        y = nan_out(t, n)
        qmm.qmm_gemm(M, pack_mxfp4(w), t, n, d, dev(x), y, ws)
        torch.cuda.synchronize()
        y = host_u16(y)
        yr, ar = oracle.gemm_mxfp4(x, w.codes, w.e8m0)
    assert_parity(y, yr, ar, f"gemm largest d {fmt} {t}x{n}x{d}")


@pytest.mark.parametrize("fmt,d", [(A, 20480), (M, 20480), (M, 65504)])
def test_grouped_long_reduction(fmt, d):
    """Grouped matmul and grouped GEMV over a long reduction axis (40 or 128
    slabs, MXFP4 ending in a narrow slab): segments of 0, 1, 5 and 70 rows."""
    say("grouped long d", fmt, d)
    n, n_exp, t = 96, 3, 80
    ws_ = [synth.affine_weights(950 + e, n, d) if fmt == A else rand_mxfp4(950 + e, n, d) for e in range(n_exp)]
    stk, size = stack(fmt, ws_)
    x = synth.activations(951, synth.S_X, t, d)
    sizes = [0, 1, 5, 70]
    seg_expert = [2, 0, 1, 2]
    seg_offsets = np.concatenate([[0], np.cumsum(sizes)])
    rng = np.random.default_rng(952)
    row_index = np.concatenate([np.sort(rng.choice(t, sz, replace=False)) for sz in sizes]).astype(np.int32)
    deq = (lambda e: oracle.dequant_affine(ws_[e].codes, ws_[e].scale, ws_[e].bias)) if fmt == A else \
          (lambda e: oracle.dequant_mxfp4(ws_[e].codes, ws_[e].e8m0))
    yr, ar = oracle.grouped(x, row_index, seg_expert, seg_offsets, deq)
    y = run_grouped(fmt, stk, size, n_exp, n, d, x, seg_expert, seg_offsets, row_index, max(sizes))
    assert_parity(y, yr, ar, f"grouped long d fmt={fmt} d={d}")
    # one row per segment: the grouped GEMV on the same weights
    seg1 = [0, 2, 1]
    off1 = np.arange(4)
    rows1 = np.asarray([3, 77, 40], np.int32)
    yr1, ar1 = oracle.grouped(x, rows1, seg1, off1, deq)
    y1 = run_grouped(fmt, stk, size, n_exp, n, d, x, seg1, off1, rows1, 1)
    assert_parity(y1, yr1, ar1, f"grouped GEMV long d fmt={fmt} d={d}")


@pytest.mark.parametrize("seed", range(16))
def test_gemm_random_shapes(seed):
    """Seeded random shapes across the GEMM's paths, two per (path, format):
    the GEMV (t = 1), the split-K kernel (2 <= t <= 64 with a workspace), for
    the same t without one the MXFP4 multi-row kernel (t <= 8 where its LDS
    holds the rows) or tile kernel (affine weights always take their
    workspace), and t > 64 with a workspace (the tile kernel, split along K
    when its tiles are few); d a multiple of 512 or ending in a narrow slab
    (MXFP4 also in a half K step), n and t ragged."""
    rng = np.random.default_rng(900 + seed)
    fmt = A if (seed // 4) % 2 == 0 else M
    kind = seed % 4
    g = 64 if fmt == A else 32
    d = int(rng.integers(1, 41)) * g
    n = int(rng.integers(1, 700))
    t = [1, int(rng.integers(2, 65)), int(rng.integers(2, 65)), int(rng.integers(65, 400))][kind]
    use_ws = kind in (1, 3) or fmt == A
    say("gemm random", seed, "fmt", fmt, "t n d", t, n, d, "ws", use_ws)
    x = synth.activations(9000 + seed, synth.S_X, t, d)
    if fmt == A:
        w = synth.affine_weights(9100 + seed, n, d)
        packed = pack_affine(w)
        yr, ar = oracle.gemm_affine(x, w.codes, w.scale, w.bias)
    else:
        w = rand_mxfp4(9100 + seed, n, d)
        packed = pack_mxfp4(w)
        yr, ar = oracle.gemm_mxfp4(x, w.codes, w.e8m0)
    need = qmm.qmm_workspace_bytes(fmt, t, n, d)
    ws = guarded((max(need, 4) // 4,), float("nan"), torch.float32) if use_ws and need else None
    y = nan_out(t, n)
    qmm.qmm_gemm(fmt, packed, t, n, d, dev(x), y, ws)
    torch.cuda.synchronize()
    assert_parity(host_u16(y), yr, ar, f"gemm random {seed}: fmt {fmt} {t}x{n}x{d} ws {use_ws}")


def test_mxfp4_e8m0_range_limits():
    """E8M0 252 (the largest exponent at which every MXFP4 weight is a finite
    bf16): the GEMV, the multi-row, tile and split-K GEMMs and the grouped
    kernels all pass parity, with activations small enough that the outputs
    stay finite.  E8M0 253 with codes of magnitude 4 and 6 (weights of 2^128
    and 1.5·2^128, beyond bf16 and fp32): the GEMV, which scales its fp32
    chunk sums, still passes; the MFMA paths, whose operands are bf16 weights,
    cannot represent that row (its values are recorded, not checked) and pass
    on the others."""
    say("mxfp4 E8M0 252 / 253")
    n, d, t = 40, 128, 3
    w = rand_mxfp4(9400, n, d)
    w.e8m0[:] = 252
    x = synth.bf16_bits(oracle.bf16_to_f64(synth.activations(9401, synth.S_X, t, d)) * 2.0 ** -20)
    p = pack_mxfp4(w)
    yr, ar = oracle.gemm_mxfp4(x, w.codes, w.e8m0)
    assert np.all(np.isfinite(yr)) and np.max(np.abs(yr)) > 2.0 ** 100
    assert_parity(run_gemv(M, p, w, x[0]), yr[0], ar[0], "gemv E8M0 252")
    assert_parity(run_gemm_multi_row(M, p, n, d, x), yr, ar, "gemm multi-row E8M0 252")
    assert_parity(run_gemm_tile(M, p, n, d, x), yr, ar, "gemm tile E8M0 252")
    assert_parity(run_gemm_split(M, p, n, d, x), yr, ar, "gemm split-k E8M0 252")
    stk, size = stack(M, [w])
    yg = run_grouped(M, stk, size, 1, n, d, x, [0], [0, t], np.arange(t), t)
    assert_parity(yg, yr, ar, "grouped E8M0 252")
    # row 0: every code of magnitude 4 or 6 (codes 6, 7, 14, 15), exponent 253
    w.e8m0[:] = 200
    w.e8m0[0, :] = 253
    w.codes[0, :] = np.array([0x76, 0xEF], np.uint8)[np.arange(d // 2) % 2]
    p = pack_mxfp4(w)
    yr, ar = oracle.gemm_mxfp4(x, w.codes, w.e8m0)
    assert np.all(np.isfinite(yr))
    assert_parity(run_gemv(M, p, w, x[0]), yr[0], ar[0], "gemv E8M0 253")
    for name, run in (("multi-row", run_gemm_multi_row), ("tile", run_gemm_tile), ("split-k", run_gemm_split)):
        yg = run(M, p, n, d, x)
        say(f"gemm {name} E8M0 253 row 0 (weights beyond bf16, not checked):",
            oracle.bf16_to_f64(yg[:, 0]).tolist(), "exact:", yr[:, 0].tolist())
        assert_parity(yg[:, 1:], yr[:, 1:], ar[:, 1:], f"gemm {name} E8M0 253, other rows")


def halfway_affine(n, d):
    """Affine weights that bf16 cannot hold: every group has scale 2^-8 and
    bias 1, so w = 1 + q·2^-8 lies exactly halfway between two bf16 numbers
    for odd q; round-to-nearest-even takes q ≡ 1 (mod 4) down and q ≡ 3
    (mod 4) up by 2^-8.  Row r holds q_dn = 1 + 4·(r % 4) on the first 32
    codes of each group and q_up = 3 + 4·(r // 4 % 4) on the last 32."""
    g = d // 64
    scale = np.full((n, g), 0x3B80, np.uint16)   # 2^-8
    bias = np.full((n, g), 0x3F80, np.uint16)    # 1.0
    q = np.empty((n, d), np.uint32)
    r = np.arange(n)
    q_dn, q_up = 1 + 4 * (r % 4), 3 + 4 * (r // 4 % 4)
    first = (np.arange(d) % 64) < 32
    q[:, first] = q_dn[:, None]
    q[:, ~first] = q_up[:, None]
    codes = np.zeros((n, d // 8), np.uint32)
    for j in range(8):
        codes |= q[:, j::8] << np.uint32(4 * j)
    return synth.Affine(codes, scale, bias), q_dn, q_up


def halfway_x(t, d):
    """x = +1 on each group's first 32 codes and -1 on its last 32, row t
    scaled by 2^(t % 5 - 2): every bf16 rounding of those weights would move
    the sum the same way."""
    sign = np.where((np.arange(d) % 64) < 32, 1.0, -1.0)
    return synth.bf16_bits(sign[None, :] * (2.0 ** (np.arange(t) % 5 - 2))[:, None])


@pytest.mark.parametrize("t,n,d", [(1, 300, 1024), (8, 300, 1024), (20, 300, 1024), (40, 300, 1024),
                                   (100, 600, 1024), (130, 300, 576), (300, 520, 5120), (2048, 4352, 512),
                                   (8, 9000, 1024), (16, 8200, 2048)])
def test_affine_weights_not_rounded(t, n, d):
    """Weights exactly halfway between two bf16 numbers, activations signed so
    that rounding them would add up: bf16 operands land at 1.94x the
    tolerance.  Every affine matmul path (GEMV, multi-row kernel, few-row
    kernel with one, two and four row blocks, tile kernel split and unsplit)
    must stay within it."""
    say("affine halfway weights", t, n, d)
    w, q_dn, q_up = halfway_affine(n, d)
    x = halfway_x(t, d)
    yr, ar = oracle.gemm_affine(x, w.codes, w.scale, w.bias)
    # the oracle, hand-worked: 32 codes of q_dn minus 32 of q_up per group
    want = (2.0 ** (np.arange(t) % 5 - 2))[:, None] * (d // 64) * 32 * (q_dn - q_up)[None, :] * 2.0 ** -8
    assert np.array_equal(yr, want)
    p = pack_affine(w)
    y = run_gemv(A, p, w, x[0])[None, :] if t == 1 else run_gemm(A, p, n, d, x)
    assert_parity(y, yr, ar, f"affine halfway {t}x{n}x{d}")


def test_grouped_affine_weights_not_rounded():
    """The same halfway weights through the routed-expert grouped kernels
    (matmul path, and the SwiGLU variant's gate and up halves)."""
    n, d = 256, 1024
    w, _, _ = halfway_affine(n, d)
    stk, size = stack(A, [w, w])
    x = halfway_x(45, d)
    seg_expert, seg_offsets = [1, 0], [0, 5, 45]
    rows = np.arange(45)
    yr, ar = oracle.gemm_affine(x, w.codes, w.scale, w.bias)
    y = run_grouped(A, stk, size, 2, n, d, x, seg_expert, seg_offsets, rows, 40)
    assert_parity(y, yr, ar, "grouped affine halfway")
    h = run_grouped_swiglu(A, stk, size, 2, n, d, x, seg_expert, seg_offsets, rows, 40)
    assert_swiglu(h, yr, ar, n // 2, "grouped swiglu affine halfway")


def test_gemm_integer_exact():
    say("gemm integer exact")
    rng = np.random.default_rng(6)
    t, n, d = 260, 300, 1024
    w = integer_affine(22, n, d)
    x = synth.bf16_bits(rng.integers(-3, 4, size=(t, d)).astype(float))
    yr, _ = oracle.gemm_affine(x, w.codes, w.scale, w.bias)
    assert np.all(np.abs(yr) < 2 ** 24)
    y = run_gemm(A, pack_affine(w), n, d, x)
    assert np.array_equal(y, oracle.f64_to_bf16_bits(yr))


def run_gemm_split(fmt, packed, n, d, x_bits):
    """qmm_gemm on the few-row split-K kernel (2 <= t <= 64; forced, since a
    wide enough matrix or few enough MXFP4 rows would take the multi-row
    kernel), with its workspace NaN-filled first: its contents on entry must
    not matter."""
    qmm.qmm_set_kernel(qmm.QMM_KERNEL_FEW_ROW)
    try:
        t = x_bits.shape[0]
        need = qmm.qmm_workspace_bytes(fmt, t, n, d)
        assert need == -(-d // 512) * t * n * 4
        ws = guarded((need // 4,), float("nan"), torch.float32)
        y = nan_out(t, n)
        qmm.qmm_gemm(fmt, packed, t, n, d, dev(x_bits), y, ws)
        torch.cuda.synchronize()
    finally:
        qmm.qmm_set_kernel(qmm.QMM_KERNEL_AUTO)
    return host_u16(y)


@pytest.mark.parametrize("t,n,d", [(2, 5, 64), (2, 300, 512), (3, 257, 1088), (16, 1000, 1024),
                                   (17, 256, 576), (33, 300, 2048), (64, 520, 640), (48, 77, 5120)])
def test_gemm_split_k_affine(t, n, d):
    say("gemm split-k affine", t, n, d)
    w = synth.affine_weights(5100 + n, n, d)
    x = synth.activations(6100 + t, synth.S_X, t, d)
    y = run_gemm_split(A, pack_affine(w), n, d, x)
    yr, ar = oracle.gemm_affine(x, w.codes, w.scale, w.bias)
    assert_parity(y, yr, ar, f"gemm split-k affine {t}x{n}x{d}")


@pytest.mark.parametrize("t,n,d,elo,ecount", [(2, 7, 32, 118, 9), (5, 300, 96, 118, 9),
                                              (16, 257, 3584, 118, 9), (64, 130, 1056, 100, 50)])
def test_gemm_split_k_mxfp4(t, n, d, elo, ecount):
    say("gemm split-k mxfp4", t, n, d)
    w = rand_mxfp4(7100 + n, n, d, elo, ecount)
    x = synth.activations(8100 + t, synth.S_X, t, d)
    y = run_gemm_split(M, pack_mxfp4(w), n, d, x)
    yr, ar = oracle.gemm_mxfp4(x, w.codes, w.e8m0)
    assert_parity(y, yr, ar, f"gemm split-k mxfp4 {t}x{n}x{d}")


@pytest.mark.parametrize("fmt,t,n,d", [(A, 65, 4096, 5120), (M, 192, 12288, 5120)])
def test_tile_split_depends_on_shape_only(fmt, t, n, d):
    """The tile GEMM splits along K into the planes the workspace layout
    reserves for the shape (eight; four where eight and the other regions
    would pass the 64 MiB of the allocation-free scratch), whatever the size
    of the buffer passed: the workspace asked for, a larger one and the
    allocation-free call give the same bits, and they meet the oracle."""
    say("tile split by shape", fmt, t, n, d)
    x = synth.activations(7300 + t, synth.S_X, t, d)
    if fmt == A:
        w = synth.affine_weights(7400 + n, n, d)
        p = pack_affine(w)
        yr, ar = oracle.gemm_affine(x, w.codes, w.scale, w.bias)
    else:
        w = rand_mxfp4(7400 + n, n, d)
        p = pack_mxfp4(w)
        yr, ar = oracle.gemm_mxfp4(x, w.codes, w.e8m0)
    need = qmm.qmm_workspace_bytes(fmt, t, n, d)
    base = (-(-t * d * 2 // 256) * 256 + -(-t * 4 // 256) * 256 + -(-n * 4 // 256) * 256) if fmt == A else 0
    planes = (need - base) // (t * n * 4)
    assert planes == (8 if base + 8 * t * n * 4 <= 64 << 20 else 4), planes
    outs = []
    for extra in (0, 32 << 20):
        ws = guarded(((need + extra) // 4,), float("nan"), torch.float32)
        y = nan_out(t, n)
        qmm.qmm_gemm(fmt, p, t, n, d, dev(x), y, ws)
        torch.cuda.synchronize()
        outs.append(host_u16(y))
    y = nan_out(t, n)
    qmm.qmm_gemm_noalloc(fmt, p, t, n, d, dev(x), y)
    torch.cuda.synchronize()
    outs.append(host_u16(y))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
    assert_parity(outs[0], yr, ar, f"tile split by shape fmt={fmt} {t}x{n}x{d}")


def run_gemm_ws(fmt, packed, n, d, x_bits):
    """qmm_gemm given the workspace qmm_workspace_bytes asks for (NaN-filled)."""
    t = x_bits.shape[0]
    need = qmm.qmm_workspace_bytes(fmt, t, n, d)
    assert need > 0
    ws = guarded((need // 4,), float("nan"), torch.float32)
    y = nan_out(t, n)
    qmm.qmm_gemm(fmt, packed, t, n, d, dev(x_bits), y, ws)
    torch.cuda.synchronize()
    return host_u16(y)


@pytest.mark.parametrize("fmt,t,n,d", [(A, 65, 300, 1024), (A, 128, 1000, 2048), (M, 200, 700, 3072),
                                       (A, 256, 4352, 1024), (M, 97, 257, 1536)])
def test_gemm_tile_split_k(fmt, t, n, d):
    """t > 64 with few tiles: the tile kernel split along K into 2, 3 or 4
    fp32 planes (ragged t and n, both formats), summed in order."""
    say("gemm tile split-k", fmt, t, n, d)
    x = synth.activations(6400 + t, synth.S_X, t, d)
    if fmt == A:
        w = synth.affine_weights(5400 + n, n, d)
        y = run_gemm_ws(A, pack_affine(w), n, d, x)
        yr, ar = oracle.gemm_affine(x, w.codes, w.scale, w.bias)
    else:
        w = rand_mxfp4(7400 + n, n, d)
        y = run_gemm_ws(M, pack_mxfp4(w), n, d, x)
        yr, ar = oracle.gemm_mxfp4(x, w.codes, w.e8m0)
    assert_parity(y, yr, ar, f"gemm tile split-k {fmt} {t}x{n}x{d}")


def test_gemm_tile_split_k_integer_exact():
    """Integer weights and activations through the split tile kernel: exact."""
    say("gemm tile split-k integer exact")
    rng = np.random.default_rng(17)
    t, n, d = 130, 300, 2048
    w = integer_affine(24, n, d)
    x = synth.bf16_bits(rng.integers(-3, 4, size=(t, d)).astype(float))
    yr, _ = oracle.gemm_affine(x, w.codes, w.scale, w.bias)
    assert np.all(np.abs(yr) < 2 ** 24)
    y = run_gemm_ws(A, pack_affine(w), n, d, x)
    assert np.array_equal(y, oracle.f64_to_bf16_bits(yr))


def test_gemm_split_k_integer_exact():
    """Integer weights and activations: every slab's partial and their sum are
    integers below 2^24, so the split-K path must match bit for bit."""
    say("gemm split-k integer exact")
    rng = np.random.default_rng(16)
    t, n, d = 20, 300, 1088
    w = integer_affine(23, n, d)
    x = synth.bf16_bits(rng.integers(-3, 4, size=(t, d)).astype(float))
    yr, _ = oracle.gemm_affine(x, w.codes, w.scale, w.bias)
    assert np.all(np.abs(yr) < 2 ** 24)
    y = run_gemm_split(A, pack_affine(w), n, d, x)
    assert np.array_equal(y, oracle.f64_to_bf16_bits(yr))


def test_gemm_split_k_decode_batch_full():
    """A batch of 8 decode rows against the whole 13824 x 5120 decode matrix,
    every output checked."""
    say("gemm split-k 8x13824x5120")
    cfg = synth.CONFIGS[1]
    n, d = cfg["n"], cfg["d"]
    w = synth.affine_weights(synth.seed_of(1), n, d)
    x = synth.activations(synth.seed_of(1), synth.S_X, 8, d, sub=3)
    y = run_gemm_split(A, pack_affine(w), n, d, x)
    yr, ar = oracle.gemm_affine(x, w.codes, w.scale, w.bias)
    assert_parity(y, yr, ar, "gemm split-k 8x13824x5120")


def test_gemm_prefill_workload_full():
    """2048 x 5120 x 13824 in the benchmark's launch configuration, every one of
    the 28.3 M outputs against the oracle (fp64, in row chunks)."""
    say("gemm affine 2048x13824x5120 full")
    cfg = synth.CONFIGS[2]
    t, n, d = cfg["t"], cfg["n"], cfg["d"]
    w = synth.affine_weights(synth.seed_of(2), n, d)
    x = synth.activations(synth.seed_of(2), synth.S_X, t, d)
    y = run_gemm(A, pack_affine(w), n, d, x)
    w_hat = oracle.dequant_affine(w.codes, w.scale, w.bias)
    worst, checked = 0.0, 0
    for r0 in range(0, t, 512):
        yr, ar = oracle.matmul(x[r0:r0 + 512], w_hat)
        r = oracle.check(y[r0:r0 + 512], yr, ar)
        assert r["ok"], (r0, r)
        worst, checked = max(worst, r["max_ratio"]), checked + r["n"]
    say("gemm 2048x13824x5120 full", dict(n=checked, max_ratio=worst))
    assert checked == t * n


# ---------------------------------------------------------------------------
# Kernel override (qmm_set_kernel): each matmul kernel forced in turn
# ---------------------------------------------------------------------------

@pytest.fixture
def kernel_auto_after():
    yield
    qmm.qmm_set_kernel(qmm.QMM_KERNEL_AUTO)


FORCED = (qmm.QMM_KERNEL_AUTO, qmm.QMM_KERNEL_TILE, qmm.QMM_KERNEL_TILE_UNSPLIT, qmm.QMM_KERNEL_FEW_ROW,
          qmm.QMM_KERNEL_MULTI_ROW)


def mrow_lds_bytes(fmt, t, d):
    """LDS of the multi-row kernel's workgroup: the rows padded to whole
    512-code slabs (one more, of zeros, for affine weights with t <= 8), the
    affine group sums of 16 rows, 6 KiB of partials."""
    rs = -(-d // 512) * 512
    rows = t + (1 if fmt == A and t <= 8 else 0)
    return rows * rs * 2 + ((rs // 64) * 16 * 4 if fmt == A else 0) + 6 * 1024


def kernel_takes(k, fmt, t, d):
    """Whether a forced kernel setting takes qmm_gemm of this shape."""
    if k == qmm.QMM_KERNEL_FEW_ROW:
        return 2 <= t <= 64
    if k == qmm.QMM_KERNEL_MULTI_ROW:
        return 2 <= t <= 16 and mrow_lds_bytes(fmt, t, d) <= 160 * 1024 or 17 <= t <= 64
    return True


def run_gemm_forced(kernel, fmt, packed, n, d, x_bits):
    """qmm_gemm under a forced kernel, with the workspace qmm_workspace_bytes
    reports under that setting (NaN-filled), none if it reports 0."""
    qmm.qmm_set_kernel(kernel)
    t = x_bits.shape[0]
    need = qmm.qmm_workspace_bytes(fmt, t, n, d)
    ws = guarded((need // 4,), float("nan"), torch.float32) if need else None
    y = nan_out(t, n)
    qmm.qmm_gemm(fmt, packed, t, n, d, dev(x_bits), y, ws)
    torch.cuda.synchronize()
    return host_u16(y)


@pytest.mark.parametrize("fmt,t,n,d", [(A, 1, 300, 1024), (A, 4, 300, 1024), (M, 4, 257, 1536),
                                       (A, 64, 520, 2048), (M, 70, 300, 1024), (A, 130, 300, 2048),
                                       (M, 1, 130, 576)])
def test_forced_kernels_integer_exact(fmt, t, n, d, kernel_auto_after):
    """Integer weights (affine scale 1 bias 0; MXFP4 with E8M0 127) and
    integer activations: every sum is exact in fp32, so the GEMV, the few-row
    kernel, the multi-row kernel and the tile kernel (split along K or not)
    must all return the oracle's sums rounded to bf16, bit for bit.  The
    few-row and multi-row kernels refuse t = 1 and t > 64."""
    say("forced kernels integer exact", fmt, t, n, d)
    rng = np.random.default_rng(40 + t)
    x = synth.bf16_bits(rng.integers(-3, 4, size=(t, d)).astype(float))
    if fmt == A:
        w = integer_affine(60 + t, n, d)
        p = pack_affine(w)
        yr, _ = oracle.gemm_affine(x, w.codes, w.scale, w.bias)
    else:
        w = rand_mxfp4(60 + t, n, d, 127, 1)
        p = pack_mxfp4(w)
        yr, _ = oracle.gemm_mxfp4(x, w.codes, w.e8m0)
    assert np.all(np.abs(yr) < 2 ** 24)
    want = oracle.f64_to_bf16_bits(yr)
    for k in FORCED:
        if not kernel_takes(k, fmt, t, d):
            qmm.qmm_set_kernel(k)
            assert qmm.qmm_workspace_bytes(fmt, t, n, d) == 0
            with pytest.raises(qmm.QmmError) as ei:
                qmm.qmm_gemm(fmt, p, t, n, d, dev(x), nan_out(t, n), None)
            assert ei.value.status == 4, ei.value   # QMM_E_UNSUPPORTED
            continue
        y = run_gemm_forced(k, fmt, p, n, d, x)
        assert np.array_equal(y, want), f"kernel setting {k}"


@pytest.mark.parametrize("fmt,t,n,d", [(A, 48, 1000, 1024), (M, 33, 300, 3584), (A, 200, 520, 2048),
                                       (A, 3, 259, 576), (M, 12, 700, 2048), (M, 64, 1100, 5120),
                                       (A, 17, 700, 4096)])
def test_forced_kernels_parity(fmt, t, n, d, kernel_auto_after):
    """Random weights and activations under every kernel setting that takes
    the shape, each within the oracle's bound."""
    say("forced kernels parity", fmt, t, n, d)
    x = synth.activations(6700 + t, synth.S_X, t, d)
    if fmt == A:
        w = synth.affine_weights(5700 + n, n, d)
        p = pack_affine(w)
        yr, ar = oracle.gemm_affine(x, w.codes, w.scale, w.bias)
    else:
        w = rand_mxfp4(7700 + n, n, d)
        p = pack_mxfp4(w)
        yr, ar = oracle.gemm_mxfp4(x, w.codes, w.e8m0)
    for k in FORCED:
        if not kernel_takes(k, fmt, t, d):
            continue
        y = run_gemm_forced(k, fmt, p, n, d, x)
        assert_parity(y, yr, ar, f"forced kernel {k} fmt={fmt} {t}x{n}x{d}")


# ---------------------------------------------------------------------------
# Multi-row GEMV (2 <= t <= 16, no workspace)
# ---------------------------------------------------------------------------

def run_gemm_multi_row(fmt, packed, n, d, x_bits):
    """qmm_gemm with the multi-row kernel forced: no workspace."""
    qmm.qmm_set_kernel(qmm.QMM_KERNEL_MULTI_ROW)
    try:
        t = x_bits.shape[0]
        assert qmm.qmm_workspace_bytes(fmt, t, n, d) == 0
        y = nan_out(t, n)
        qmm.qmm_gemm(fmt, packed, t, n, d, dev(x_bits), y, None)
        torch.cuda.synchronize()
    finally:
        qmm.qmm_set_kernel(qmm.QMM_KERNEL_AUTO)
    return host_u16(y)


def auto_picks_multi_row(fmt, t, n, d):
    """The library's own choice for qmm_gemm (no workspace asked for)."""
    if not kernel_takes(qmm.QMM_KERNEL_MULTI_ROW, fmt, t, d):
        return False
    if t > 16:
        return d <= 2048 or (n >= 6912 and d <= 5120) or n >= 10240
    if d <= 3072:
        return True
    return n >= 5120 or t <= 8 if fmt == M else n >= 8192


# launch shapes covered: 1 to 8 column waves per workgroup; the slabs shared
# by 4, 2 or 1 wave groups; more workgroups than 256 CUs (n > 32768); one
# narrow slab; a narrow last slab; n not a multiple of 4 or 16; t from 2 to 16
# (the most rows each format's LDS holds at d = 5120); the decode matrix
MULTI_ROW_SHAPES = [(A, 2, 5, 64), (A, 3, 300, 320), (A, 16, 1000, 1024), (A, 8, 257, 1088),
                    (A, 5, 4099, 5184), (A, 14, 13824, 5120), (A, 8, 13824, 5120), (A, 7, 16385, 2048),
                    (A, 2, 33000, 640), (A, 16, 3000, 4096), (A, 11, 9001, 1536), (A, 4, 27648, 2048),
                    (M, 2, 7, 32), (M, 5, 300, 96), (M, 16, 257, 3584), (M, 15, 13824, 5120),
                    (M, 9, 16500, 1056), (M, 4, 1024, 5152), (M, 13, 33001, 512), (M, 8, 5121, 2080),
                    (M, 3, 32768, 1024)]


@pytest.mark.parametrize("fmt,t,n,d", MULTI_ROW_SHAPES)
def test_gemm_multi_row(fmt, t, n, d, kernel_auto_after):
    """The multi-row kernel against the oracle; where the library picks it by
    itself, the call without a forced setting gives the same bits."""
    say("gemm multi-row", fmt, t, n, d)
    x = synth.activations(9100 + t, synth.S_X, t, d)
    if fmt == A:
        w = synth.affine_weights(9200 + n, n, d)
        p = pack_affine(w)
        yr, ar = oracle.gemm_affine(x, w.codes, w.scale, w.bias)
    else:
        w = rand_mxfp4(9300 + n, n, d)
        p = pack_mxfp4(w)
        yr, ar = oracle.gemm_mxfp4(x, w.codes, w.e8m0)
    y = run_gemm_multi_row(fmt, p, n, d, x)
    assert_parity(y, yr, ar, f"gemm multi-row fmt={fmt} {t}x{n}x{d}")
    if auto_picks_multi_row(fmt, t, n, d):
        assert qmm.qmm_workspace_bytes(fmt, t, n, d) == 0
        ya = nan_out(t, n)
        qmm.qmm_gemm(fmt, p, t, n, d, dev(x), ya, None)
        torch.cuda.synchronize()
        assert np.array_equal(host_u16(ya), y)


@pytest.mark.parametrize("fmt,t,n,d", [(A, 8, 13824, 5120), (A, 16, 3000, 4096), (A, 13, 1000, 5184),
                                       (M, 15, 13824, 5120), (M, 6, 20000, 1536)])
def test_gemm_multi_row_integer_exact(fmt, t, n, d, kernel_auto_after):
    """Integer weights and activations: the multi-row kernel returns the
    oracle's exact sums rounded to bf16, bit for bit the few-row kernel's."""
    say("gemm multi-row integer exact", fmt, t, n, d)
    rng = np.random.default_rng(70 + t)
    x = synth.bf16_bits(rng.integers(-3, 4, size=(t, d)).astype(float))
    if fmt == A:
        w = integer_affine(80 + t, n, d)
        p = pack_affine(w)
        yr, _ = oracle.gemm_affine(x, w.codes, w.scale, w.bias)
    else:
        w = rand_mxfp4(80 + t, n, d, 127, 1)
        p = pack_mxfp4(w)
        yr, _ = oracle.gemm_mxfp4(x, w.codes, w.e8m0)
    assert np.all(np.abs(yr) < 2 ** 24)
    want = oracle.f64_to_bf16_bits(yr)
    assert np.array_equal(run_gemm_multi_row(fmt, p, n, d, x), want)
    assert np.array_equal(run_gemm_forced(qmm.QMM_KERNEL_FEW_ROW, fmt, p, n, d, x), want)


@pytest.mark.parametrize("seed", range(12))
def test_gemm_multi_row_random_shapes(seed, kernel_auto_after):
    """Seeded random shapes on the multi-row kernel (forced): t from 2 to 16,
    n from 1 to 40000 (one to eight column waves per workgroup, one or two
    workgroups per CU), d any multiple of the group up to what the rows' LDS
    allows, both formats."""
    rng = np.random.default_rng(1900 + seed)
    fmt = A if seed % 2 == 0 else M
    g = 64 if fmt == A else 32
    t = int(rng.integers(2, 17))
    n = int(rng.choice([rng.integers(1, 300), rng.integers(300, 9000), rng.integers(9000, 40001)]))
    d = g * int(rng.integers(1, 6144 // g + 1))
    while not kernel_takes(qmm.QMM_KERNEL_MULTI_ROW, fmt, t, d):
        d -= g * 8 if d > g * 8 else 0
        t = max(2, t - 1)
    say("gemm multi-row random", seed, "fmt", fmt, "t n d", t, n, d)
    x = synth.activations(1910 + seed, synth.S_X, t, d)
    if fmt == A:
        w = synth.affine_weights(1920 + seed, n, d)
        p = pack_affine(w)
        yr, ar = oracle.gemm_affine(x, w.codes, w.scale, w.bias)
    else:
        w = rand_mxfp4(1920 + seed, n, d)
        p = pack_mxfp4(w)
        yr, ar = oracle.gemm_mxfp4(x, w.codes, w.e8m0)
    y = run_gemm_multi_row(fmt, p, n, d, x)
    assert_parity(y, yr, ar, f"gemm multi-row random {seed}: fmt {fmt} {t}x{n}x{d}")


# the streaming form (17 <= t <= 64, two to four row blocks of 16): one
# narrow slab; a narrow last slab; fewer than 16 columns; a workgroup of one
# to four column waves; more workgroups than 256 CUs (n > 16384); t just past
# each row block; the decode matrix at 32, 48 and 64 rows; d = 65536
MULTI_ROW_STREAM_SHAPES = [(A, 17, 300, 64), (A, 32, 1000, 1088), (A, 64, 13824, 5120), (A, 48, 4099, 5184),
                           (A, 33, 33000, 640), (A, 50, 3, 128), (A, 40, 16385, 2048), (M, 17, 7, 32),
                           (M, 64, 257, 3584), (M, 49, 13824, 5120), (M, 63, 16500, 1056), (M, 20, 5121, 2080),
                           (M, 32, 13824, 5120), (M, 35, 40000, 96),
                           # the largest reduction axis (128 slabs; MXFP4 ending in a narrow slab)
                           (A, 64, 130, 65536), (A, 17, 700, 65536), (M, 33, 97, 65504)]


@pytest.mark.parametrize("fmt,t,n,d", MULTI_ROW_STREAM_SHAPES)
def test_gemm_multi_row_streamed(fmt, t, n, d, kernel_auto_after):
    """The multi-row kernel's streaming form against the oracle; where the
    library picks it by itself, the call without a forced setting gives the
    same bits."""
    say("gemm multi-row streamed", fmt, t, n, d)
    x = synth.activations(9600 + t, synth.S_X, t, d)
    if fmt == A:
        w = synth.affine_weights(9700 + n, n, d)
        p = pack_affine(w)
        yr, ar = oracle.gemm_affine(x, w.codes, w.scale, w.bias)
    else:
        w = rand_mxfp4(9800 + n, n, d)
        p = pack_mxfp4(w)
        yr, ar = oracle.gemm_mxfp4(x, w.codes, w.e8m0)
    y = run_gemm_multi_row(fmt, p, n, d, x)
    assert_parity(y, yr, ar, f"gemm multi-row streamed fmt={fmt} {t}x{n}x{d}")
    if auto_picks_multi_row(fmt, t, n, d):
        assert qmm.qmm_workspace_bytes(fmt, t, n, d) == 0
        ya = nan_out(t, n)
        qmm.qmm_gemm(fmt, p, t, n, d, dev(x), ya, None)
        torch.cuda.synchronize()
        assert np.array_equal(host_u16(ya), y)


@pytest.mark.parametrize("fmt,t,n,d", [(A, 64, 13824, 5120), (A, 37, 1000, 5184), (M, 64, 13824, 5120),
                                       (M, 18, 6000, 1568)])
def test_gemm_multi_row_streamed_integer_exact(fmt, t, n, d, kernel_auto_after):
    """Integer weights and activations through the streaming form: the
    oracle's exact sums rounded to bf16, bit for bit the few-row kernel's."""
    say("gemm multi-row streamed integer exact", fmt, t, n, d)
    rng = np.random.default_rng(170 + t)
    x = synth.bf16_bits(rng.integers(-3, 4, size=(t, d)).astype(float))
    if fmt == A:
        w = integer_affine(180 + t, n, d)
        p = pack_affine(w)
        yr, _ = oracle.gemm_affine(x, w.codes, w.scale, w.bias)
    else:
        w = rand_mxfp4(180 + t, n, d, 127, 1)
        p = pack_mxfp4(w)
        yr, _ = oracle.gemm_mxfp4(x, w.codes, w.e8m0)
    assert np.all(np.abs(yr) < 2 ** 24)
    want = oracle.f64_to_bf16_bits(yr)
    assert np.array_equal(run_gemm_multi_row(fmt, p, n, d, x), want)
    assert np.array_equal(run_gemm_forced(qmm.QMM_KERNEL_FEW_ROW, fmt, p, n, d, x), want)


@pytest.mark.parametrize("seed", range(8))
def test_gemm_multi_row_streamed_random_shapes(seed, kernel_auto_after):
    """Seeded random shapes on the streaming form: t from 17 to 64, n from 1
    to 40000, d any multiple of the group up to 6144, both formats."""
    rng = np.random.default_rng(2900 + seed)
    fmt = A if seed % 2 == 0 else M
    g = 64 if fmt == A else 32
    t = int(rng.integers(17, 65))
    n = int(rng.choice([rng.integers(1, 300), rng.integers(300, 9000), rng.integers(9000, 40001)]))
    d = g * int(rng.integers(1, 6144 // g + 1))
    say("gemm multi-row streamed random", seed, "fmt", fmt, "t n d", t, n, d)
    x = synth.activations(2910 + seed, synth.S_X, t, d)
    if fmt == A:
        w = synth.affine_weights(2920 + seed, n, d)
        p = pack_affine(w)
        yr, ar = oracle.gemm_affine(x, w.codes, w.scale, w.bias)
    else:
        w = rand_mxfp4(2920 + seed, n, d)
        p = pack_mxfp4(w)
        yr, ar = oracle.gemm_mxfp4(x, w.codes, w.e8m0)
    y = run_gemm_multi_row(fmt, p, n, d, x)
    assert_parity(y, yr, ar, f"gemm multi-row streamed random {seed}: fmt {fmt} {t}x{n}x{d}")


def test_gemm_multi_row_repeated_and_shrinking(kernel_auto_after):
    """Calls in a row on one stream, the second with fewer rows and columns
    and a shorter reduction: nothing carries over between launches."""
    say("gemm multi-row repeated")
    for t, n, d in [(12, 13824, 5120), (3, 999, 1088), (12, 13824, 5120), (64, 13824, 5120), (20, 999, 1088)]:
        x = synth.activations(9400 + t, synth.S_X, t, d)
        w = synth.affine_weights(9500 + n, n, d)
        y = run_gemm_multi_row(A, pack_affine(w), n, d, x)
        yr, ar = oracle.gemm_affine(x, w.codes, w.scale, w.bias)
        assert_parity(y, yr, ar, f"gemm multi-row repeated {t}x{n}x{d}")


# ---------------------------------------------------------------------------
# Grouped (routed experts)
# ---------------------------------------------------------------------------

def stack(fmt, weights):
    size = qmm.qmm_packed_bytes(fmt, weights[0].n, weights[0].d)
    out = torch.empty(size * len(weights), dtype=torch.uint8, device=DEV)
    for e, w in enumerate(weights):
        p = pack_affine(w) if fmt == A else pack_mxfp4(w)
        out[e * size:(e + 1) * size].copy_(p)
    return out, size


def run_grouped(fmt, stk, stride, n_exp, n, d, x_bits, seg_expert, seg_offsets, row_index, max_rows):
    m_total = int(seg_offsets[-1])
    y = nan_out(m_total, n)
    qmm.qmm_grouped_gemm(fmt, stk, stride, n_exp, n, d, dev(x_bits), x_bits.shape[0],
                         dev(np.asarray(row_index, np.int32)), dev(np.asarray(seg_expert, np.int32)),
                         dev(np.asarray(seg_offsets, np.int32)), len(seg_expert), m_total, max_rows, y)
    torch.cuda.synchronize()
    return host_u16(y)


@pytest.mark.parametrize("fmt,d", [(A, 256), (M, 256), (A, 576), (M, 1056)])
def test_grouped_gemm_small(fmt, d):
    """Segments of 0 .. 130 rows (two 64-row passes), n not a multiple of the
    column tile; d = 256 is one narrow slab, 576 / 1056 add a narrow last slab
    after full ones (metadata read per slab in both shapes)."""
    say("grouped small", fmt, d)
    n, n_exp, t = 300, 5, 140
    ws = [synth.affine_weights(900 + e, n, d) if fmt == A else rand_mxfp4(900 + e, n, d) for e in range(n_exp)]
    stk, size = stack(fmt, ws)
    x = synth.activations(901, synth.S_X, t, d)
    sizes = [0, 1, 17, 64, 65, 130]
    seg_expert = [4, 0, 2, 1, 3, 2]
    seg_offsets = np.concatenate([[0], np.cumsum(sizes)])
    rng = np.random.default_rng(8)
    row_index = np.concatenate([np.sort(rng.choice(t, s, replace=False)) for s in sizes]).astype(np.int32)
    deq = (lambda e: oracle.dequant_affine(ws[e].codes, ws[e].scale, ws[e].bias)) if fmt == A else \
          (lambda e: oracle.dequant_mxfp4(ws[e].codes, ws[e].e8m0))
    yr, ar = oracle.grouped(x, row_index, seg_expert, seg_offsets, deq)
    for max_rows in (max(sizes), 1):      # MFMA path, then the GEMV path on the same table
        y = run_grouped(fmt, stk, size, n_exp, n, d, x, seg_expert, seg_offsets, row_index, max_rows)
        assert_parity(y, yr, ar, f"grouped fmt={fmt} d={d} max_rows={max_rows}")


@pytest.mark.parametrize("fmt", [A, M])
def test_grouped_forced_matmul_on_one_row_segments(fmt, kernel_auto_after):
    """One row per segment takes the grouped GEMV; forced, the matmul kernel
    takes the same table.  Integer weights and activations: both exact."""
    say("grouped forced matmul", fmt)
    n, d, n_exp, t = 300, 1024, 6, 16
    ws = [integer_affine(930 + e, n, d) if fmt == A else rand_mxfp4(930 + e, n, d, 127, 1) for e in range(n_exp)]
    stk, size = stack(fmt, ws)
    rng = np.random.default_rng(31)
    x = synth.bf16_bits(rng.integers(-3, 4, size=(t, d)).astype(float))
    seg_expert = [5, 0, 3, 2, 1]
    seg_offsets = np.arange(len(seg_expert) + 1)
    row_index = np.asarray([7, 0, 15, 3, 9], np.int32)
    deq = (lambda e: oracle.dequant_affine(ws[e].codes, ws[e].scale, ws[e].bias)) if fmt == A else \
          (lambda e: oracle.dequant_mxfp4(ws[e].codes, ws[e].e8m0))
    yr, _ = oracle.grouped(x, row_index, seg_expert, seg_offsets, deq)
    assert np.all(np.abs(yr) < 2 ** 24)
    want = oracle.f64_to_bf16_bits(yr)
    for k in (qmm.QMM_KERNEL_AUTO, qmm.QMM_KERNEL_GROUPED_MATMUL):
        qmm.qmm_set_kernel(k)
        y = run_grouped(fmt, stk, size, n_exp, n, d, x, seg_expert, seg_offsets, row_index, 1)
        assert np.array_equal(y, want), f"kernel setting {k}"


def run_grouped_order(fmt, stk, stride, n_exp, n, d, x_bits, seg_expert, seg_offsets, max_rows):
    """The grouped call with row_index NULL: grouped row r reads x row r."""
    m_total = int(seg_offsets[-1])
    y = nan_out(m_total, n)
    qmm.qmm_grouped_gemm(fmt, stk, stride, n_exp, n, d, dev(x_bits), x_bits.shape[0], None,
                         dev(np.asarray(seg_expert, np.int32)), dev(np.asarray(seg_offsets, np.int32)),
                         len(seg_expert), m_total, max_rows, y)
    torch.cuda.synchronize()
    return host_u16(y)


# a bound of 2 .. 8 rows per segment takes the multi-row kernel (one
# workgroup per 128-column block and segment, each segment's rows gathered
# into LDS, a longer segment in several passes); shapes:
# one narrow slab and a narrow last slab, n not a multiple of 64, affine with
# 8 rows or fewer (two groups per MFMA) and with more, the decode experts
GROUPED_MR_SHAPES = [(A, 300, 1024), (A, 257, 576), (M, 300, 2080), (M, 6144, 3584), (A, 129, 64), (M, 97, 32)]


@pytest.mark.parametrize("fmt,n,d", GROUPED_MR_SHAPES)
def test_grouped_multi_row(fmt, n, d, kernel_auto_after):
    """Segments of 0 .. 16 rows through the multi-row kernel (bounds of 2 to
    8 rows per pass) against the oracle: a segment longer than the bound
    takes several passes of that many rows; also with the rows in order
    (row_index NULL), and the matmul kernel forced on the same table."""
    say("grouped multi-row", fmt, n, d)
    n_exp, t = 6, 48
    ws = [synth.affine_weights(960 + e, n, d) if fmt == A else rand_mxfp4(960 + e, n, d) for e in range(n_exp)]
    stk, size = stack(fmt, ws)
    x = synth.activations(961, synth.S_X, t, d)
    sizes = [0, 1, 3, 16, 5, 0, 2, 9]
    seg_expert = [4, 0, 2, 5, 3, 1, 2, 0]
    seg_offsets = np.concatenate([[0], np.cumsum(sizes)])
    rng = np.random.default_rng(12)
    row_index = np.concatenate([np.sort(rng.choice(t, sz, replace=False)) for sz in sizes]).astype(np.int32)
    deq = (lambda e: oracle.dequant_affine(ws[e].codes, ws[e].scale, ws[e].bias)) if fmt == A else \
          (lambda e: oracle.dequant_mxfp4(ws[e].codes, ws[e].e8m0))
    yr, ar = oracle.grouped(x, row_index, seg_expert, seg_offsets, deq)
    # a bound above 8 splits the call: segments of up to 8 rows to the
    # multi-row kernel, 9 and 16 to the matmul kernel
    for max_rows in (8, 4, 2, 16):
        y = run_grouped(fmt, stk, size, n_exp, n, d, x, seg_expert, seg_offsets, row_index, max_rows)
        assert_parity(y, yr, ar, f"grouped multi-row fmt={fmt} {n}x{d} max_rows={max_rows}")
    m_total = int(seg_offsets[-1])
    yro, aro = oracle.grouped(x[:m_total], np.arange(m_total), seg_expert, seg_offsets, deq)
    for max_rows in (8, 16):
        yo = run_grouped_order(fmt, stk, size, n_exp, n, d, x[:m_total], seg_expert, seg_offsets, max_rows)
        assert_parity(yo, yro, aro, f"grouped multi-row rows in order fmt={fmt} {n}x{d} max_rows={max_rows}")
    qmm.qmm_set_kernel(qmm.QMM_KERNEL_GROUPED_MATMUL)
    y = run_grouped(fmt, stk, size, n_exp, n, d, x, seg_expert, seg_offsets, row_index, 16)
    assert_parity(y, yr, ar, f"grouped matmul forced fmt={fmt} {n}x{d}")


@pytest.mark.parametrize("fmt", [A, M])
def test_grouped_multi_row_integer_exact(fmt, kernel_auto_after):
    """Integer weights and activations: the multi-row kernel (true and
    understated bound), the split call (the 12-row segment to the matmul
    kernel, the others to the multi-row kernel) and the matmul kernel alone
    return the oracle's exact sums rounded to bf16, bit for bit."""
    say("grouped multi-row integer exact", fmt)
    n, d, n_exp, t = 200, 1536, 4, 30
    ws = [integer_affine(970 + e, n, d) if fmt == A else rand_mxfp4(970 + e, n, d, 127, 1) for e in range(n_exp)]
    stk, size = stack(fmt, ws)
    rng = np.random.default_rng(33)
    x = synth.bf16_bits(rng.integers(-3, 4, size=(t, d)).astype(float))
    sizes = [7, 0, 12, 3]
    seg_expert = [3, 1, 0, 2]
    seg_offsets = np.concatenate([[0], np.cumsum(sizes)])
    row_index = rng.integers(0, t, int(seg_offsets[-1])).astype(np.int32)
    deq = (lambda e: oracle.dequant_affine(ws[e].codes, ws[e].scale, ws[e].bias)) if fmt == A else \
          (lambda e: oracle.dequant_mxfp4(ws[e].codes, ws[e].e8m0))
    yr, _ = oracle.grouped(x, row_index, seg_expert, seg_offsets, deq)
    assert np.all(np.abs(yr) < 2 ** 24)
    want = oracle.f64_to_bf16_bits(yr)
    for k, max_rows in ((qmm.QMM_KERNEL_AUTO, 8), (qmm.QMM_KERNEL_AUTO, 5), (qmm.QMM_KERNEL_AUTO, 12),
                        (qmm.QMM_KERNEL_GROUPED_MATMUL, 12)):
        qmm.qmm_set_kernel(k)
        y = run_grouped(fmt, stk, size, n_exp, n, d, x, seg_expert, seg_offsets, row_index, max_rows)
        assert np.array_equal(y, want), f"kernel setting {k}, max_rows {max_rows}"


# ---------------------------------------------------------------------------
# expert FFN: gate_up with the SwiGLU activation, down on the activated rows,
# weighted combine back to the tokens
# ---------------------------------------------------------------------------

def run_grouped_swiglu(fmt, stk, stride, n_exp, n, d, x_bits, seg_expert, seg_offsets, row_index, max_rows):
    m_total = int(seg_offsets[-1])
    h = nan_out(m_total, n // 2)
    qmm.qmm_grouped_gemm_swiglu(fmt, stk, stride, n_exp, n, d, dev(x_bits), x_bits.shape[0],
                                dev(np.asarray(row_index, np.int32)), dev(np.asarray(seg_expert, np.int32)),
                                dev(np.asarray(seg_offsets, np.int32)), len(seg_expert), m_total, max_rows, h)
    torch.cuda.synchronize()
    return host_u16(h)


def assert_swiglu(h_bits, y_ref, a_ref, n_inter, what):
    """h = silu(g)·u checked against the fp64 SwiGLU of the fp64 gate_up
    result, within the bound that the gate and up values' own acceptance
    (2e-3·A + 1e-5 each) carries through silu and the product, then the one
    bf16 rounding."""
    tol_y = oracle.REL_TOL * np.asarray(a_ref, np.float64) + oracle.ABS_TOL
    h_ref = oracle.swiglu(y_ref, n_inter)
    tol_h = oracle.swiglu_tolerance(y_ref, tol_y, n_inter)
    r = oracle.check(h_bits, h_ref, tol_h, rel=1.0, abs_=0.0)
    say(what, {k: r[k] for k in ("n", "n_fail", "max_ratio", "max_abs")})
    assert r["ok"], (what, r)


@pytest.mark.parametrize("fmt,d", [(A, 256), (M, 256), (A, 576), (M, 1056)])
def test_grouped_swiglu_small(fmt, d, kernel_auto_after):
    """gate_up stacks of 600 rows (300 gate, 300 up: the last 128-column tile
    is partial), segments of 0 .. 130 rows, narrow last slabs; the true bound
    splits the segments (up to 8 rows to the multi-row kernel, the rest to
    the matmul kernel), bounds of 8 and 1 take the multi-row kernel alone (a
    longer segment in passes of 8 or 2 rows), and the matmul kernel forced
    takes them all."""
    say("grouped swiglu small", fmt, d)
    n, n_exp, t = 600, 5, 140
    ws = [synth.affine_weights(960 + e, n, d) if fmt == A else rand_mxfp4(960 + e, n, d) for e in range(n_exp)]
    stk, size = stack(fmt, ws)
    x = synth.activations(961, synth.S_X, t, d)
    sizes = [0, 1, 17, 64, 5, 65, 130, 8]
    seg_expert = [4, 0, 2, 1, 0, 3, 2, 4]
    seg_offsets = np.concatenate([[0], np.cumsum(sizes)])
    rng = np.random.default_rng(9)
    row_index = np.concatenate([np.sort(rng.choice(t, s, replace=False)) for s in sizes]).astype(np.int32)
    deq = (lambda e: oracle.dequant_affine(ws[e].codes, ws[e].scale, ws[e].bias)) if fmt == A else \
          (lambda e: oracle.dequant_mxfp4(ws[e].codes, ws[e].e8m0))
    yr, ar = oracle.grouped(x, row_index, seg_expert, seg_offsets, deq)
    for k, max_rows in ((qmm.QMM_KERNEL_AUTO, max(sizes)), (qmm.QMM_KERNEL_AUTO, 8), (qmm.QMM_KERNEL_AUTO, 1),
                        (qmm.QMM_KERNEL_GROUPED_MATMUL, max(sizes))):
        qmm.qmm_set_kernel(k)
        h = run_grouped_swiglu(fmt, stk, size, n_exp, n, d, x, seg_expert, seg_offsets, row_index, max_rows)
        assert_swiglu(h, yr, ar, n // 2, f"swiglu fmt={fmt} d={d} kernel={k} max_rows={max_rows}")


def test_grouped_rows_in_order():
    """row_index NULL: grouped row r reads x row r, also with one row per
    segment (which then takes the matmul kernel)."""
    say("grouped rows in order")
    n, d, n_exp = 200, 1056, 3
    ws = [rand_mxfp4(970 + e, n, d) for e in range(n_exp)]
    stk, size = stack(M, ws)
    sizes = [3, 0, 40, 1]
    seg_expert = [2, 1, 0, 2]
    seg_offsets = np.concatenate([[0], np.cumsum(sizes)])
    m_total = int(seg_offsets[-1])
    x = synth.activations(971, synth.S_X, m_total, d)
    deq = lambda e: oracle.dequant_mxfp4(ws[e].codes, ws[e].e8m0)
    yr, ar = oracle.grouped(x, np.arange(m_total), seg_expert, seg_offsets, deq)
    for max_rows in (40, 1):
        y = nan_out(m_total, n)
        qmm.qmm_grouped_gemm(M, stk, size, n_exp, n, d, dev(x), m_total, None, dev(np.asarray(seg_expert, np.int32)),
                             dev(np.asarray(seg_offsets, np.int32)), len(seg_expert), m_total, max_rows, y)
        torch.cuda.synchronize()
        assert_parity(host_u16(y), yr, ar, f"grouped rows in order max_rows={max_rows}")


def run_combine(o_bits, topk, weights, seg_offsets, row_index, d):
    t, k = topk.shape
    out = nan_out(t, d)
    qmm.qmm_moe_combine(dev(o_bits), o_bits.shape[0], d, t, k, dev(np.asarray(topk, np.int32)),
                        dev(np.asarray(weights, np.float32)), weights.shape[1],
                        dev(np.asarray(seg_offsets, np.int32)), dev(np.asarray(row_index, np.int32)), out)
    torch.cuda.synchronize()
    return host_u16(out)


@pytest.mark.parametrize("t,ne,k,d", [(40, 20, 4, 96), (7, 65, 64, 8), (130, 300, 16, 1032)])
def test_combine_small(t, ne, k, d):
    """The combine against the oracle's on the same inputs: the fp64 routing's
    tables and fp32 weights, random bf16 expert outputs."""
    say("combine", t, ne, k, d)
    x, r, bias = synth.router_inputs(7300 + t, t=t, d=64, experts=ne)
    sig = oracle.route_scores(x, r, None)[0].astype(np.float32)
    tk = oracle.topk(oracle.route_scores(x, r, bias)[0], k)
    offs, rows = oracle.group(tk, ne)
    o = synth.activations(7301 + t, synth.S_X, t * k, d)
    out = run_combine(o, tk, sig, offs, rows, d)
    yr, ar = oracle.combine(oracle.bf16_to_f64(o), tk, sig.astype(np.float64), offs, rows)
    assert_parity(out, yr, ar, f"combine t={t} ne={ne} k={k} d={d}")


@pytest.mark.parametrize("t,ne,k,d", [(1000, 5, 3, 64), (700, 20, 16, 40), (300, 40, 24, 16),
                                      (300, 40, 40, 24)])
def test_combine_long_segments(t, ne, k, d):
    """Segments of tens to hundreds of rows, with 64, 16, 8 and 4 lanes
    searching each slot's row (k = 3, 16, 24, 40): several narrowing rounds
    before the last one.  Then one token is taken out of the longest segment
    (the rows after it move up): that token's outputs are NaN, every other
    token's unchanged."""
    say("combine long segments", t, ne, k, d)
    x, r, bias = synth.router_inputs(7500 + k, t=t, d=64, experts=ne)
    sig = oracle.route_scores(x, r, None)[0].astype(np.float32)
    tk = oracle.topk(oracle.route_scores(x, r, bias)[0], k)
    offs, rows = oracle.group(tk, ne)
    lens = np.diff(offs)
    assert lens.max() > 64
    o = synth.activations(7501 + k, synth.S_X, t * k, d)
    out = run_combine(o, tk, sig, offs, rows, d)
    yr, ar = oracle.combine(oracle.bf16_to_f64(o), tk, sig.astype(np.float64), offs, rows)
    assert_parity(out, yr, ar, f"combine long t={t} ne={ne} k={k} d={d}")

    e = int(np.argmax(lens))
    pos = int(offs[e]) + int(lens[e]) // 2   # a token in the middle of the longest segment
    gone = int(rows[pos])
    rows2 = np.delete(rows, pos)
    o2 = np.delete(o, pos, axis=0)
    offs2 = offs.copy()
    offs2[e + 1:] -= 1
    out2 = oracle.bf16_to_f64(run_combine(o2, tk, sig, offs2, rows2, d))
    assert np.all(np.isnan(out2[gone]))
    keep = np.arange(t) != gone
    assert np.array_equal(out2[keep], oracle.bf16_to_f64(out)[keep], equal_nan=True)


def test_combine_missing_row_gives_nan():
    say("combine missing row")
    tk = np.array([[0, 1], [1, 0]])
    offs = np.array([0, 1, 3])               # expert 0 lists token 0 only
    rows = np.array([0, 0, 1])
    w = np.full((2, 2), 0.5, np.float32)
    o = synth.activations(7400, synth.S_X, 3, 16)
    out = oracle.bf16_to_f64(run_combine(o, tk, w, offs, rows, 16))
    assert np.all(np.isfinite(out[0])) and np.all(np.isnan(out[1]))


def test_grouped_invalid_entries_give_nan():
    say("grouped invalid entries")
    n, d, n_exp, t = 40, 128, 2, 8
    ws = [rand_mxfp4(950 + e, n, d) for e in range(n_exp)]
    stk, size = stack(M, ws)
    x = synth.activations(951, synth.S_X, t, d)
    seg_expert = [0, 7, 1]                  # expert 7 does not exist
    seg_offsets = [0, 2, 4, 6]
    row_index = [1, 2, 3, 4, 5, 99]         # row 99 does not exist
    for max_rows in (2, 1):
        y = run_grouped(M, stk, size, n_exp, n, d, x, seg_expert, seg_offsets, row_index, max_rows)
        yf = oracle.bf16_to_f64(y)
        assert np.all(np.isnan(yf[2:4])) and np.all(np.isnan(yf[5]))
        assert np.all(np.isfinite(yf[0:2])) and np.all(np.isfinite(yf[4]))
    # a bound of 16 splits the segments (10 and 9 rows to the matmul kernel,
    # 3 and 2 to the multi-row kernel), with and without the activation:
    # each kernel marks its own segments' bad rows
    seg_expert = [0, 7, 1, -1]
    seg_offsets = [0, 10, 19, 22, 24]
    row_index = [0, 1, 2, 3, 99, 5, 6, 7, 1, 2] + [0] * 9 + [3, 100, 5] + [1, 2]
    bad = np.zeros(24, bool)
    bad[[4, 20, 22, 23]] = True
    bad[10:19] = True
    # (outputs start at zero, so a NaN row is one a kernel wrote)
    for glu in (False, True):
        call = qmm.qmm_grouped_gemm_swiglu if glu else qmm.qmm_grouped_gemm
        y = torch.zeros(24, n // 2 if glu else n, dtype=torch.int16, device="cuda")
        call(M, stk, size, n_exp, n, d, dev(x), t, dev(np.asarray(row_index, np.int32)),
             dev(np.asarray(seg_expert, np.int32)), dev(np.asarray(seg_offsets, np.int32)), 4, 24, 16, y)
        torch.cuda.synchronize()
        yf = oracle.bf16_to_f64(host_u16(y))
        assert np.all(np.isnan(yf[bad])) and np.all(np.isfinite(yf[~bad])), f"glu={glu}"
        assert np.count_nonzero(yf[~bad]) > 0.9 * yf[~bad].size, f"glu={glu}: good rows written"


def make_expert_stack(which, n_exp):
    import synth.gpu as sg
    n, d = (6144, 3584) if which == "gate_up" else (3584, 3072)
    size = qmm.qmm_packed_bytes(M, n, d)
    out = torch.empty(size * n_exp, dtype=torch.uint8, device=DEV)
    sg.expert_stack(synth.seed_of(3), which, n_exp,
                    lambda c, e, ptr: qmm.qmm_pack(M, n, d, c, e, None, ptr), size, size, out)
    return out, size


@pytest.fixture(scope="module")
def expert_stacks():
    say("building 896-expert stacks on the GPU")
    gu = make_expert_stack("gate_up", 896)
    dn = make_expert_stack("down", 896)
    torch.cuda.synchronize()
    yield gu, dn
    del gu, dn
    torch.cuda.empty_cache()


def test_moe_decode_workload_full(expert_stacks):
    """16 routed experts, gate_up on x then down on a seeded z per expert,
    every output against the oracle."""
    say("moe decode grouped gemv full")
    (gu, gsz), (dn, dsz) = expert_stacks
    seed = synth.seed_of(3)
    experts = synth.draw_experts(seed, 16, 896, 0)
    x = synth.activations(seed, synth.S_X, 1, 3584)
    z = synth.activations(seed, synth.S_Z, 16, 3072)
    seg_offsets = np.arange(17)
    y1 = run_grouped(M, gu, gsz, 896, 6144, 3584, x, experts, seg_offsets, np.zeros(16, np.int32), 1)
    y2 = run_grouped(M, dn, dsz, 896, 3584, 3072, z, experts, seg_offsets, np.arange(16), 1)
    for i, e in enumerate(experts):
        g = synth.expert_gate_up(seed, int(e))
        yr, ar = oracle.gemm_mxfp4(x, g.codes, g.e8m0)
        assert_parity(y1[i], yr[0], ar[0], f"gate_up expert {e}")
        dw = synth.expert_down(seed, int(e))
        yr, ar = oracle.gemm_mxfp4(z[i:i + 1], dw.codes, dw.e8m0)
        assert_parity(y2[i], yr[0], ar[0], f"down expert {e}")


def grouped_columns(n, tile=256, extra=80, seed=0):
    """Output columns checked on every segment: the first and last column of
    each tile of the grouped kernel, and `extra` more at random."""
    edges = {c for t0 in range(0, n, tile) for c in (t0, min(t0 + tile, n) - 1)}
    rng = np.random.default_rng(seed)
    return np.array(sorted(edges | set(rng.choice(n, extra, replace=False).tolist())), np.int64)


def check_all_segments(y, x_rows, seg_expert, seg_offsets, row_index, rows_fn, n, what, full_count=32):
    """Every row of every segment of a grouped output y [m_total, n] against the
    oracle on a column sample (tile edges included), regenerating only those
    weight rows of each expert (rows_fn(e, cols); cols None for the whole
    matrix); `full_count` segments spread over the size range are checked on
    all n columns.  Returns the number of outputs checked."""
    sizes = np.diff(np.asarray(seg_offsets))
    active = np.nonzero(sizes)[0]
    cols = grouped_columns(n)
    by_size = active[np.argsort(sizes[active], kind="stable")]
    full = set(by_size[np.linspace(0, len(by_size) - 1, min(full_count, len(by_size))).astype(int)].tolist())
    checked, worst = 0, 0.0
    for s_ in active:
        r0, r1 = int(seg_offsets[s_]), int(seg_offsets[s_ + 1])
        e = int(seg_expert[s_])
        xs = x_rows[np.asarray(row_index)[r0:r1]]
        c = np.arange(n) if s_ in full else cols
        wr = rows_fn(e, None if s_ in full else c)
        yr, ar = oracle.matmul(xs, oracle.dequant_mxfp4(wr.codes, wr.e8m0))
        r = oracle.check(y[r0:r1][:, c], yr, ar)
        assert r["ok"], (what, s_, e, r1 - r0, r)
        checked, worst = checked + r["n"], max(worst, r["max_ratio"])
    say(what, dict(segments=len(active), full_segments=len(full), columns_sampled=len(cols),
                   outputs_checked=checked, max_ratio=worst))
    return checked


def test_moe_prefill_workload_all_segments(expert_stacks):
    """512 tokens routed top-16 over 896 experts, one grouped call; every row of
    all active segments is checked against the oracle on a column sample that
    holds each 256-column tile's first and last column, and 32 segments across
    the size range on all 6144 columns."""
    say("moe prefill grouped gemm, all segments")
    (gu, gsz), _ = expert_stacks
    seed = synth.seed_of(4)
    xb, rb, bias = synth.router_inputs(seed)
    rt = oracle.route(xb, rb, bias)
    # the prefill workload reuses the decode workload's expert weights
    y = run_grouped(M, gu, gsz, 896, 6144, 3584, xb, rt.seg_expert, rt.seg_offsets, rt.row_index,
                    rt.max_seg_rows)
    assert not np.any(y == NAN16)
    rows_fn = lambda e, c: (synth.expert_gate_up(synth.seed_of(3), e) if c is None
                            else synth.expert_gate_up_rows(synth.seed_of(3), e, c))
    n_checked = check_all_segments(y, xb, rt.seg_expert, rt.seg_offsets, rt.row_index, rows_fn, 6144,
                                   "moe prefill grouped gemm")
    assert n_checked > 8192 * 128


def test_bitwise_deterministic():
    say("determinism")
    w = synth.affine_weights(31, 1000, 5120)
    p = pack_affine(w)
    x = synth.activations(32, synth.S_X, 300, 5120)
    a = run_gemm(A, p, 1000, 5120, x)
    b = run_gemm(A, p, 1000, 5120, x)
    assert np.array_equal(a, b)
    a = run_gemv(A, p, w, x[0])
    b = run_gemv(A, p, w, x[0])
    assert np.array_equal(a, b)


def test_profile_events_time_the_kernel():
    say("profile events")
    import bench
    hev = bench.HipEvents()
    w = synth.affine_weights(41, 4096, 4096)
    p = pack_affine(w)
    x = dev(synth.activations(42, synth.S_X, 1, 4096))
    y = nan_out(4096)
    a, b = hev.new(), hev.new()
    qmm.qmm_profile_next(a, b)
    qmm.qmm_gemv(A, p, 4096, 4096, x, y)
    torch.cuda.synchronize()
    ms = hev.ms(a, b)
    hev.close()
    assert 0.0 < ms < 5.0
    assert not np.any(host_u16(y) == NAN16)


def test_stream_read_reads_every_byte():
    """The read-ceiling kernel: XOR of its per-workgroup words equals the
    XOR of the buffer (ragged size: not a multiple of the grid's stride)."""
    say("stream read")
    rng = np.random.default_rng(77)
    words = rng.integers(0, 2 ** 32, size=(39_851_008 // 4 + 4,), dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).to(DEV)
    sink = torch.zeros(2048, dtype=torch.int32, device=DEV)
    qmm.qmm_stream_read(buf, words.size * 4, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(words)


# ---------------------------------------------------------------------------
# Router
# ---------------------------------------------------------------------------

def run_route(x_bits, r_bits, bias, k):
    t, d = x_bits.shape
    ne = r_bits.shape[0]
    scores = guarded((t, ne), float("nan"), torch.float32)
    topk = guarded((t, k), -1, torch.int32)
    seg_e = guarded((ne,), -1, torch.int32)
    seg_o = guarded((ne + 1,), -1, torch.int32)
    rows = guarded((t * k,), -1, torch.int32)
    qmm.qmm_route(dev(x_bits), t, d, dev(r_bits), ne, None if bias is None else dev(bias), k,
                  scores, topk, seg_e, seg_o, rows)
    torch.cuda.synchronize()
    return (scores.cpu().numpy().astype(np.float64), topk.cpu().numpy(), seg_e.cpu().numpy(),
            seg_o.cpu().numpy(), rows.cpu().numpy())


def check_route(x, r, bias, k, what):
    """Scores are the bare sigmoid (the routing weights); the choice is made on
    sigmoid + bias, whose fp32 sum adds one rounding of at most 2^-24·|sum| to
    the score's bound, well inside its 1e-6 absolute term."""
    s_gpu, tk, seg_e, seg_o, rows = run_route(x, r, bias, k)
    sig_ref, a_ref = oracle.route_scores(x, r, None)
    sel_ref, _ = oracle.route_scores(x, r, bias)
    delta = oracle.route_score_bound(a_ref, x.shape[1])
    err = np.abs(s_gpu - sig_ref)
    say(what, dict(max_err=float(err.max()), max_err_over_bound=float((err / delta).max())))
    assert np.all(err <= delta), what
    res = oracle.check_topk(tk, sel_ref, delta)
    say(what, {kk: res[kk] for kk in ("n_bad", "rows_equal_to_fp64_choice", "rows")})
    assert res["ok"], (what, res)
    offs, ridx = oracle.group(tk, r.shape[0])        # exact, given the GPU's own choice
    assert np.array_equal(seg_e, np.arange(r.shape[0])), what
    assert np.array_equal(seg_o, offs) and np.array_equal(rows, ridx), what
    return tk, seg_o, rows


@pytest.mark.parametrize("t,d,ne,k", [(48, 256, 96, 16), (70, 136, 100, 5), (1, 8, 1, 1),
                                      (130, 512, 1024, 64), (9, 1024, 65, 64),
                                      (1000, 64, 96, 16),     # t*k = 16000: tables held in registers, 2 passes
                                      (1100, 64, 120, 16)])   # t*k = 17600: tables streamed, 3 passes
def test_route_small(t, d, ne, k):
    say("route", t, d, ne, k)
    x, r, bias = synth.router_inputs(7000 + t, t=t, d=d, experts=ne)
    check_route(x, r, bias, k, f"route {t}x{d} over {ne} top-{k}")


def test_route_ties_go_to_the_lower_id():
    """Experts with identical router rows and bias score identically (same
    arithmetic in every lane), so the choice among them is fixed by the id."""
    say("route ties")
    x, r, bias = synth.router_inputs(7100, t=20, d=128, experts=40)
    r = r.copy()
    bias = bias.copy()
    for e in (7, 19, 33):                      # three copies of expert 3
        r[e] = r[3]
        bias[e] = bias[3]
    s_gpu, tk, _, _, _ = run_route(x, r, bias, 12)
    assert np.all(s_gpu[:, [7, 19, 33]] == s_gpu[:, [3]])
    for row in tk:
        picked = [e for e in row.tolist() if e in (3, 7, 19, 33)]
        assert picked == sorted(picked)          # listed in id order
        assert picked == [3, 7, 19, 33][:len(picked)]   # the lowest ids are the ones taken


def test_route_non_finite_scores_rank_last():
    """A bias of -inf or NaN: those experts come after every finite score, -inf
    before NaN, each class in id order -- over 100 experts, so two keys per
    lane, and k = 64 reaches into all three classes."""
    say("route non-finite")
    x, r, bias = synth.router_inputs(7200, t=24, d=256, experts=100)
    ids = np.random.default_rng(7201).permutation(100)
    fin, ninf, nan = ids[:44], ids[44:54], ids[54:]
    bias = bias.copy()
    bias[fin] = 2.0 * np.arange(44, 0, -1)         # spaced wider than the sigmoid's range
    bias[ninf] = -np.inf
    bias[nan] = np.nan
    s_gpu, tk, seg_e, seg_o, rows = run_route(x, r, bias, 64)
    assert np.all(np.isfinite(s_gpu))   # the weights are the bare sigmoid; the bias only selects
    want = fin.tolist() + sorted(ninf.tolist()) + sorted(nan.tolist())[:10]
    assert all(row.tolist() == want for row in tk)
    sref = oracle.route_scores(x, r, bias)[0]
    assert all(row.tolist() == want for row in oracle.topk(sref, 64))
    offs, rws = oracle.group(tk, 100)
    assert np.array_equal(seg_e, np.arange(100))
    assert np.array_equal(seg_o, offs) and np.array_equal(rows, rws)


def test_moe_prefill_expert_ffn(expert_stacks):
    """The routed prefill workload through the whole expert FFN on the GPU:
    route -> gate_up with SwiGLU -> down on the activated rows -> combine.
    Each stage is checked against the oracle on the GPU's own inputs to that
    stage (sampled experts for the matmuls, every output of the combine)."""
    say("moe prefill expert ffn")
    (gu, gsz), (dn, dsz) = expert_stacks
    xb, rb, bias = synth.router_inputs(synth.seed_of(4))
    t, ne, k = 512, 896, 16
    s_gpu, tk, seg_e, seg_o, rows = run_route(xb, rb, bias, k)
    m_total = t * k
    h = run_grouped_swiglu(M, gu, gsz, ne, 6144, 3584, xb, seg_e, seg_o, rows, 512)
    o = nan_out(m_total, 3584)
    qmm.qmm_grouped_gemm(M, dn, dsz, ne, 3584, 3072, dev(h), m_total, None, dev(seg_e), dev(seg_o), ne,
                         m_total, 512, o)
    torch.cuda.synchronize()
    o = host_u16(o)
    out = run_combine(o, tk, s_gpu.astype(np.float32), seg_o, rows, 3584)
    sizes = np.diff(seg_o)
    active = np.nonzero(sizes)[0]
    rng = np.random.default_rng(12)
    for e in sorted({int(active[np.argmax(sizes[active])]), *rng.choice(active, 3, replace=False).tolist()}):
        r0, r1 = int(seg_o[e]), int(seg_o[e + 1])
        g = synth.expert_gate_up(synth.seed_of(3), e)
        yr, ar = oracle.gemm_mxfp4(xb[rows[r0:r1]], g.codes, g.e8m0)
        assert_swiglu(h[r0:r1], yr, ar, 3072, f"ffn gate_up+swiglu expert {e} rows {r1 - r0}")
        dw = synth.expert_down(synth.seed_of(3), e)
        yr, ar = oracle.gemm_mxfp4(h[r0:r1], dw.codes, dw.e8m0)
        assert_parity(o[r0:r1], yr, ar, f"ffn down expert {e} rows {r1 - r0}")
    yr, ar = oracle.combine(oracle.bf16_to_f64(o), tk, s_gpu, seg_o, rows)
    assert_parity(out, yr, ar, "ffn combine 512x3584")


def test_route_prefill_workload_then_grouped_gemm(expert_stacks):
    """512 tokens x 3584 routed top-16 over 896 experts on the GPU, every score
    and choice checked; the tables then drive the grouped matmul directly
    (dense segments, empty ones included), sampled against the oracle."""
    say("route prefill workload")
    (gu, gsz), _ = expert_stacks
    xb, rb, bias = synth.router_inputs(synth.seed_of(4))
    tk, seg_o, rows = check_route(xb, rb, bias, 16, "route 512x3584 over 896 top-16")
    y = run_grouped(M, gu, gsz, 896, 6144, 3584, xb, np.arange(896), seg_o, rows, 512)
    sizes = np.diff(seg_o)
    assert not np.any(y == NAN16)
    rng = np.random.default_rng(11)
    active = np.nonzero(sizes)[0]
    for e in sorted({int(active[np.argmax(sizes[active])]), *rng.choice(active, 5, replace=False).tolist()}):
        r0, r1 = int(seg_o[e]), int(seg_o[e + 1])
        g = synth.expert_gate_up(synth.seed_of(3), e)
        yr, ar = oracle.gemm_mxfp4(xb[rows[r0:r1]], g.codes, g.e8m0)
        assert_parity(y[r0:r1], yr, ar, f"routed expert {e} rows {r1 - r0}")
