"""qmm_gemm_noalloc (the split-K GEMM with its partial sums in the library's
static scratch instead of a caller workspace) against qmm_gemm given a
workspace: the same kernels in the same order, so the outputs must be bitwise
equal, and both within the oracle's tolerance.  Each case makes two calls in a
row, the second with a smaller input, so the second finds the first's partial
sums in the shared scratch."""
import sys

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import bit_weight_quantized_amd as qmm  # noqa: E402

A, M = qmm.QMM_AFFINE4_G64, qmm.QMM_MXFP4_G32
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


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    elif a.dtype == np.uint32:
        a = a.view(np.int32)
    return torch.from_numpy(a).to(DEV)


def packed_weights(fmt, seed, n, d):
    if fmt == A:
        w = synth.affine_weights(seed, n, d)
        p = torch.empty(qmm.qmm_packed_bytes(A, n, d), dtype=torch.uint8, device=DEV)
        qmm.qmm_pack(A, n, d, dev(w.codes), dev(w.scale), dev(w.bias), p)
        ref = lambda x: oracle.gemm_affine(x, w.codes, w.scale, w.bias)
    else:
        w = synth.mxfp4_weights(seed, n, d, synth.S_GU_CODES, synth.S_GU_E8M0, 0)
        p = torch.empty(qmm.qmm_packed_bytes(M, n, d), dtype=torch.uint8, device=DEV)
        qmm.qmm_pack(M, n, d, dev(w.codes), dev(w.e8m0), None, p)
        ref = lambda x: oracle.gemm_mxfp4(x, w.codes, w.e8m0)
    return p, ref


def both(fmt, p, t, n, d, x):
    """(no-alloc output, workspace output) as bf16 bits; outputs start as NaN."""
    need = qmm.qmm_workspace_bytes(fmt, t, n, d)
    assert 0 < need <= 64 << 20, need
    xd = dev(x)
    y0 = torch.full((t, n), 0x7FC0, dtype=torch.int16, device=DEV)
    qmm.qmm_gemm_noalloc(fmt, p, t, n, d, xd, y0)
    ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device=DEV)
    y1 = torch.full((t, n), 0x7FC0, dtype=torch.int16, device=DEV)
    qmm.qmm_gemm(fmt, p, t, n, d, xd, y1, ws)
    torch.cuda.synchronize()
    return y0.cpu().numpy().view(np.uint16), y1.cpu().numpy().view(np.uint16)


# (format, n, d, first t, second t): few-row split-K (16 < t <= 64 on
# matrices of under 6144 columns, and narrow affine matrices below that), the tile kernel split along K (t > 64
# with few tiles, d a multiple of 512), and the affine tile kernel unsplit
# (its fp16 activations in the scratch)
CASES = [(A, 4096, 5120, 40, 20), (M, 1000, 3584, 64, 17), (A, 4096, 3584, 12, 3),
         (A, 1000, 2048, 200, 70), (M, 700, 3072, 97, 66), (A, 4352, 1024, 2048, 300)]


@pytest.mark.parametrize("fmt,n,d,t1,t2", CASES)
def test_noalloc_matches_workspace_call(fmt, n, d, t1, t2):
    p, ref = packed_weights(fmt, 9100 + n, n, d)
    for t in (t1, t2):
        say("gemm_noalloc", "affine" if fmt == A else "mxfp4", t, n, d)
        x = synth.activations(9200 + t, synth.S_X, t, d)
        y0, y1 = both(fmt, p, t, n, d, x)
        assert np.array_equal(y0, y1), f"no-alloc differs from the workspace call at t={t}"
        yr, ar = ref(x)
        r = oracle.check(y0, yr, ar)
        say("gemm_noalloc", t, {k: r[k] for k in ("n", "n_fail", "max_ratio")})
        assert r["ok"], r


def test_noalloc_single_row_and_limit():
    n, d = 512, 256
    p, ref = packed_weights(A, 9300, n, d)
    x = synth.activations(9301, synth.S_X, 1, d)
    y = torch.full((1, n), 0x7FC0, dtype=torch.int16, device=DEV)
    qmm.qmm_gemm_noalloc(A, p, 1, n, d, dev(x), y)     # t = 1: the GEMV, no scratch
    torch.cuda.synchronize()
    yr, ar = ref(x)
    assert oracle.check(y.cpu().numpy().view(np.uint16), yr, ar)["ok"]
    # partials beyond the 64 MiB scratch are refused before any launch
    big_n, big_d = 6000, 32768
    assert qmm.qmm_workspace_bytes(A, 64, big_n, big_d) > 64 << 20
    with pytest.raises(qmm.QmmError) as ei:
        qmm.qmm_gemm_noalloc(A, 1 << 20, 64, big_n, big_d, 1 << 20, 1 << 20)
    assert ei.value.name == "QMM_E_WORKSPACE"


@pytest.mark.parametrize("fmt,n,d,t", [(A, 13824, 5120, 8), (M, 1000, 3584, 3), (M, 13824, 5120, 33),
                                       (A, 2100, 1024, 40)])
def test_noalloc_multi_row_takes_no_scratch(fmt, n, d, t):
    """Shapes on the multi-row kernel need no workspace: the allocation-free
    call runs the same kernel as qmm_gemm, bit for bit, twice in a row."""
    p, ref = packed_weights(fmt, 9400 + n, n, d)
    assert qmm.qmm_workspace_bytes(fmt, t, n, d) == 0
    x = synth.activations(9500 + t, synth.S_X, t, d)
    xd = dev(x)
    outs = []
    for _ in range(2):
        y0 = torch.full((t, n), 0x7FC0, dtype=torch.int16, device=DEV)
        qmm.qmm_gemm_noalloc(fmt, p, t, n, d, xd, y0)
        y1 = torch.full((t, n), 0x7FC0, dtype=torch.int16, device=DEV)
        qmm.qmm_gemm(fmt, p, t, n, d, xd, y1, None)
        torch.cuda.synchronize()
        outs.append((y0.cpu().numpy().view(np.uint16), y1.cpu().numpy().view(np.uint16)))
    assert all(np.array_equal(a, b) for a, b in outs) and np.array_equal(outs[0][0], outs[1][0])
    yr, ar = ref(x)
    assert oracle.check(outs[0][0], yr, ar)["ok"]
