"""C-ABI checks that need no GPU: the library loads, exports every function
include/qmm.h declares, sizes its blobs by the format arithmetic, and rejects
bad arguments on the host before any HIP call."""
import os
import re

import pytest

import bit_weight_quantized_amd as qmm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HAVE_LIB = os.path.exists(qmm.lib_path())
pytestmark = pytest.mark.skipif(not HAVE_LIB, reason="libqmm.so not built (run __graft_entry__.build())")

A, M = qmm.QMM_AFFINE4_G64, qmm.QMM_MXFP4_G32
OK, E_ARG, E_SHAPE, E_ALIGN, E_UNSUPPORTED, E_WS = 0, 1, 2, 3, 4, 5


def declared_functions():
    with open(os.path.join(ROOT, "include", "qmm.h"), encoding="utf-8") as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qmm_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = qmm.load()
    names = declared_functions()
    assert set(names) == set(qmm.EXPORTS)
    for name in names:
        assert hasattr(lib, name), name
    nm = os.popen(f"nm -D --defined-only {qmm.lib_path()}").read()
    for name in names:
        assert re.search(rf"\bT {name}\b", nm), name


def test_packed_bytes_arithmetic():
    # 256-byte header + codes + metadata, rounded to 256; payload is 36 B per 64 affine
    # weights and 17 B per 32 MXFP4 weights.
    for n, d in [(512, 256), (13824, 5120), (7, 192), (1, 64)]:
        payload = n * d // 2 + n * d // 64 * 4
        assert payload == 36 * n * d // 64
        got = qmm.qmm_packed_bytes(A, n, d)
        assert got % 256 == 0 and payload + 256 <= got < payload + 256 + 512
    assert qmm.qmm_packed_bytes(A, 13824, 5120) == 256 + 39_813_120
    for n, d in [(6144, 3584), (3584, 3072), (3, 96)]:
        payload = n * d // 2 + n * d // 32
        assert payload * 32 == 17 * n * d
        got = qmm.qmm_packed_bytes(M, n, d)
        assert got % 256 == 0 and payload + 256 <= got < payload + 256 + 512
    assert qmm.qmm_packed_bytes(M, 6144, 3584) == 256 + 11_698_176
    assert qmm.qmm_packed_bytes(M, 3584, 3072) == 256 + 5_849_088


def test_packed_bytes_rejects_bad_shapes():
    for f, n, d in [(A, 8, 96), (M, 8, 48), (A, 0, 64), (A, 8, 0), (3, 8, 64), (A, -1, 64),
                    (A, 8, 65536 + 64), (A, (1 << 28) + 1, 64)]:
        assert qmm.qmm_packed_bytes(f, n, d) == 0
    assert qmm.qmm_workspace_bytes(A, 1, 13824, 5120) == 0


def test_workspace_contract():
    # the multi-row kernel (2 <= t <= 16, rows within its LDS; any n where
    # d <= 3072, else MXFP4 from 5120 columns or up to 8 rows, affine from 8192; 17 <= t <= 64 where
    # d <= 2048, from 6912 columns while d <= 5120, from 10240 beyond) takes none
    assert qmm.qmm_workspace_bytes(A, 2, 13824, 5120) == 0
    assert qmm.qmm_workspace_bytes(A, 14, 13824, 5120) == 0
    assert qmm.qmm_workspace_bytes(M, 8, 1024, 5120) == 0
    assert qmm.qmm_workspace_bytes(M, 15, 5120, 5120) == 0
    assert qmm.qmm_workspace_bytes(A, 17, 13824, 5120) == 0
    assert qmm.qmm_workspace_bytes(M, 64, 10240, 8192) == 0
    assert qmm.qmm_workspace_bytes(A, 40, 6912, 5120) == 0
    assert qmm.qmm_workspace_bytes(A, 40, 300, 2048) == 0
    assert qmm.qmm_workspace_bytes(A, 4, 16, 64) == 0
    assert qmm.qmm_workspace_bytes(A, 16, 300, 3072) == 0
    # split-K partials of qmm_gemm for the other 2 <= t <= 64: one fp32 [t][n]
    # plane per 512-code slab of d; nothing for other t or invalid shapes
    assert qmm.qmm_workspace_bytes(A, 2, 4096, 5120) == 10 * 2 * 4096 * 4
    assert qmm.qmm_workspace_bytes(A, 15, 13824, 5120) == 10 * 15 * 13824 * 4   # 15 rows exceed its LDS
    assert qmm.qmm_workspace_bytes(M, 12, 1024, 5120) == 10 * 12 * 1024 * 4
    assert qmm.qmm_workspace_bytes(A, 16, 300, 3584) == 7 * 16 * 300 * 4
    assert qmm.qmm_workspace_bytes(A, 17, 4096, 5120) == 10 * 17 * 4096 * 4
    assert qmm.qmm_workspace_bytes(M, 64, 6911, 2560) == 5 * 64 * 6911 * 4
    assert qmm.qmm_workspace_bytes(A, 40, 6144, 4096) == 8 * 40 * 6144 * 4
    assert qmm.qmm_workspace_bytes(M, 40, 8192, 8192) == 16 * 40 * 8192 * 4
    assert qmm.qmm_workspace_bytes(M, 64, 300, 2560) == 5 * 64 * 300 * 4
    for t in (1, 2048, 300):
        assert qmm.qmm_workspace_bytes(M, t, 13824, 5120) == 0
    # affine weights through the tile kernel (t > 64): the activations as fp16,
    # one int32 exponent per row and per weight column, each region rounded up
    # to 256 bytes
    up = lambda v: -(-v // 256) * 256
    assert qmm.qmm_workspace_bytes(A, 2048, 13824, 5120) == 2048 * 5120 * 2 + 2048 * 4 + 13824 * 4
    assert qmm.qmm_workspace_bytes(A, 300, 13824, 5120) == 300 * 5120 * 2 + up(300 * 4) + 13824 * 4
    # the tile kernel split along K (up to 8 planes) while 128-row tiles would
    # cover at most half of a 256-CU chip; d a multiple of 512 only
    assert qmm.qmm_workspace_bytes(A, 65, 13824, 5120) == up(65 * 5120 * 2) + up(65 * 4) + 13824 * 4 + 8 * 65 * 13824 * 4
    assert qmm.qmm_workspace_bytes(M, 128, 8192, 5120) == 8 * 128 * 8192 * 4
    # four planes where eight (and the other regions) would pass the 64 MiB of
    # the allocation-free scratch
    assert qmm.qmm_workspace_bytes(M, 256, 13824, 5120) == 4 * 256 * 13824 * 4
    assert qmm.qmm_workspace_bytes(M, 65, 13824, 5056) == 0
    assert qmm.qmm_workspace_bytes(A, 65, 13824, 5056) == up(65 * 5056 * 2) + up(65 * 4) + 13824 * 4
    assert qmm.qmm_workspace_bytes(A, 4, 8, 96) == 0
    # optional, but one that is passed must be large enough and 16-byte aligned
    # (host validation: nothing is launched)
    lib = qmm.load()
    need = qmm.qmm_workspace_bytes(A, 4, 16, 5120)
    assert need == 10 * 4 * 16 * 4
    assert lib.qmm_gemm(A, P, 4, 16, 5120, P, P, P, need - 1, None) == E_WS
    assert "workspace" in qmm.qmm_last_error()
    assert lib.qmm_gemm(A, P, 4, 16, 5120, P, P, P + 8, need, None) == E_ALIGN
    assert lib.qmm_gemv(A, P, 16, 64, P + 1, P, P, 1, None) == E_ALIGN   # gemv ignores ws, checks x
    # affine weights with t >= 2 cannot do without it
    assert lib.qmm_gemm(A, P, 2048, 16, 64, P, P, None, 0, None) == E_WS
    assert "affine" in qmm.qmm_last_error()


def test_noalloc_limit_is_checked_on_the_host():
    # the allocation-free GEMM refuses shapes whose split-K partials exceed its
    # 64 MiB static scratch before looking up the scratch or launching anything
    lib = qmm.load()
    assert qmm.qmm_workspace_bytes(A, 64, 6000, 32768) > 64 << 20
    assert lib.qmm_gemm_noalloc(A, P, 64, 6000, 32768, P, P, None) == E_WS
    assert "64 MiB" in qmm.qmm_last_error()
    assert lib.qmm_gemm_noalloc(A, P + 8, 8, 16, 64, P, P, None) == E_ALIGN
    assert lib.qmm_gemm_noalloc(A, P, 0, 16, 64, P, P, None) == E_ARG


@pytest.fixture
def kernel_auto_after():
    yield
    qmm.qmm_set_kernel(qmm.QMM_KERNEL_AUTO)


def test_kernel_override_sizes_and_refusals(kernel_auto_after):
    """The workspace follows the forced kernel; a shape the forced kernel does
    not take is refused on the host."""
    lib = qmm.load()
    up = lambda v: -(-v // 256) * 256
    assert lib.qmm_set_kernel(6) == E_ARG and lib.qmm_set_kernel(-1) == E_ARG
    assert qmm.qmm_get_kernel() == qmm.QMM_KERNEL_AUTO
    skinny4 = 10 * 4 * 13824 * 4
    assert qmm.qmm_workspace_bytes(A, 4, 13824, 5120) == 0                 # the multi-row kernel
    tile_aff = lambda t: up(t * 5120 * 2) + up(t * 4) + 13824 * 4
    qmm.qmm_set_kernel(qmm.QMM_KERNEL_TILE)
    assert qmm.qmm_get_kernel() == qmm.QMM_KERNEL_TILE
    assert qmm.qmm_workspace_bytes(A, 4, 13824, 5120) == tile_aff(4)       # no split for t <= 64
    assert qmm.qmm_workspace_bytes(A, 1, 13824, 5120) == tile_aff(1)       # t = 1 on the tile kernel too
    assert qmm.qmm_workspace_bytes(A, 65, 13824, 5120) == tile_aff(65) + 8 * 65 * 13824 * 4
    assert qmm.qmm_workspace_bytes(M, 4, 13824, 5120) == 0
    assert lib.qmm_gemm(A, P, 1, 16, 64, P, P, None, 0, None) == E_WS     # affine tile needs one at t = 1
    qmm.qmm_set_kernel(qmm.QMM_KERNEL_TILE_UNSPLIT)
    assert qmm.qmm_workspace_bytes(A, 65, 13824, 5120) == tile_aff(65)
    assert qmm.qmm_workspace_bytes(M, 256, 13824, 5120) == 0
    qmm.qmm_set_kernel(qmm.QMM_KERNEL_FEW_ROW)
    assert qmm.qmm_workspace_bytes(A, 4, 13824, 5120) == skinny4
    assert qmm.qmm_workspace_bytes(M, 4, 13824, 5120) == skinny4
    assert qmm.qmm_workspace_bytes(A, 65, 13824, 5120) == 0
    assert lib.qmm_gemm(A, P, 65, 16, 64, P, P, P, 1 << 20, None) == E_UNSUPPORTED
    assert lib.qmm_gemm(A, P, 1, 16, 64, P, P, P, 1 << 20, None) == E_UNSUPPORTED
    assert "few-row" in qmm.qmm_last_error()
    assert lib.qmm_gemm(M, P, 4, 16, 64, P, P, None, 0, None) == E_WS     # few-row needs one for MXFP4 too
    qmm.qmm_set_kernel(qmm.QMM_KERNEL_MULTI_ROW)
    assert qmm.qmm_workspace_bytes(A, 4, 13824, 5120) == 0
    assert qmm.qmm_workspace_bytes(A, 4, 1024, 5120) == 0                  # narrow matrices too
    assert qmm.qmm_workspace_bytes(A, 17, 13824, 5120) == 0                # streamed rows
    assert qmm.qmm_workspace_bytes(M, 64, 13824, 5120) == 0
    assert qmm.qmm_workspace_bytes(A, 65, 13824, 5120) == 0                # refused below
    assert lib.qmm_gemm(A, P, 65, 16, 64, P, P, None, 0, None) == E_UNSUPPORTED
    assert "multi-row" in qmm.qmm_last_error()
    assert lib.qmm_gemm(A, P, 1, 16, 64, P, P, None, 0, None) == E_UNSUPPORTED
    assert lib.qmm_gemm(A, P, 15, 16, 5120, P, P, None, 0, None) == E_UNSUPPORTED   # rows beyond its LDS
    assert lib.qmm_gemm_noalloc(A, P, 65, 16, 64, P, P, None) == E_UNSUPPORTED
    qmm.qmm_set_kernel(qmm.QMM_KERNEL_GROUPED_MATMUL)
    assert qmm.qmm_workspace_bytes(A, 4, 13824, 5120) == 0                 # no effect on qmm_gemm
    assert qmm.qmm_workspace_bytes(A, 4, 4096, 5120) == 10 * 4 * 4096 * 4
    qmm.qmm_set_kernel(qmm.QMM_KERNEL_AUTO)
    assert qmm.qmm_workspace_bytes(A, 4, 13824, 5120) == 0
    assert qmm.qmm_workspace_bytes(A, 4, 4096, 5120) == 10 * 4 * 4096 * 4


@pytest.mark.parametrize("value,want", [("tile", 1), ("tile_unsplit", 2), ("few_row", 3),
                                        ("grouped_matmul", 4), ("4", 4), ("multi_row", 5), ("5", 5),
                                        ("auto", 0), ("", 0), ("Tile", -1), ("fast", -1), ("6", -1)])
def test_kernel_override_from_the_environment(value, want):
    """QMM_FORCE_KERNEL sets the initial value; an unknown one makes the
    matmul calls fail with QMM_E_ARG until qmm_set_kernel is called."""
    import subprocess
    import sys
    code = f"""
import bit_weight_quantized_amd as qmm
lib = qmm.load()
P = 1 << 20
assert qmm.qmm_get_kernel() == {want}, qmm.qmm_get_kernel()
if {want} < 0:
    assert qmm.qmm_workspace_bytes(1, 4, 16, 64) == 0
    assert lib.qmm_gemm(1, P, 4, 16, 64, P, P, P, 1 << 20, None) == 1
    assert "QMM_FORCE_KERNEL" in qmm.qmm_last_error()
    stride = qmm.qmm_packed_bytes(2, 16, 64)
    assert lib.qmm_grouped_gemm(2, P, stride, 1, 16, 64, P, 1, P, P, P, 1, 1, 1, P, None, 0, None) == 1
    assert "QMM_FORCE_KERNEL" in qmm.qmm_last_error()
    qmm.qmm_set_kernel(qmm.QMM_KERNEL_AUTO)
    assert qmm.qmm_get_kernel() == 0
    assert qmm.qmm_workspace_bytes(1, 4, 16, 5120) == 2560
"""
    env = dict(os.environ, QMM_FORCE_KERNEL=value)
    r = subprocess.run([sys.executable, "-c", code], env=env, cwd=ROOT, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr[-2000:]


def test_status_strings_and_version():
    assert qmm.qmm_status_string(0) == "ok"
    for s in range(1, 9):
        assert qmm.qmm_status_string(s) not in ("ok", "unknown status")
    assert qmm.qmm_status_string(99) == "unknown status"
    assert qmm.qmm_layout_version() >= 1


P = 1 << 20          # a 256-aligned fake device address: validation never dereferences it


def expect(status, fn, *args):
    with pytest.raises(qmm.QmmError) as ei:
        fn(*args)
    assert ei.value.status == status, (ei.value, qmm.qmm_last_error())


def test_validation_errors_before_any_launch():
    # every call here fails host validation; nothing reaches HIP
    expect(E_ARG, qmm.qmm_gemv, 7, P, 16, 64, P, P, None, 0)            # unknown format
    expect(E_SHAPE, qmm.qmm_gemv, A, P, 16, 96, P, P, None, 0)           # d % 64
    expect(E_SHAPE, qmm.qmm_gemv, M, P, 16, 48, P, P, None, 0)           # d % 32
    expect(E_ARG, qmm.qmm_gemv, A, P, 0, 64, P, P, None, 0)              # n = 0
    expect(E_ARG, qmm.qmm_gemv, A, None, 16, 64, P, P, None, 0)          # NULL packed
    expect(E_ARG, qmm.qmm_gemv, A, P, 16, 64, None, P, None, 0)          # NULL x
    expect(E_ALIGN, qmm.qmm_gemv, A, P + 16, 16, 64, P, P, None, 0)      # packed 256-byte
    expect(E_ALIGN, qmm.qmm_gemv, A, P, 16, 64, P + 8, P, None, 0)       # x 16-byte
    expect(E_ALIGN, qmm.qmm_gemv, A, P, 16, 64, P, P + 1, None, 0)       # y 2-byte
    expect(E_ARG, qmm.qmm_gemm, A, P, 0, 16, 64, P, P, None, 0)          # t = 0
    expect(E_SHAPE, qmm.qmm_gemm, A, P, (1 << 24) + 1, 16, 64, P, P, None, 0)
    expect(E_ARG, qmm.qmm_pack, A, 16, 64, P, P, None, P, 0)             # affine needs biases
    expect(E_ARG, qmm.qmm_pack, M, 16, 64, P, P, P, P, 0)                # MXFP4 takes none
    expect(E_ALIGN, qmm.qmm_pack, A, 16, 64, P, P, P, P + 64, 0)
    expect(E_ALIGN, qmm.qmm_pack, A, 16, 64, P + 2, P, P, P, 0)          # codes 4-byte
    expect(E_ARG, qmm.qmm_unpack, A, 16, 64, None, P, P, P, 0)
    blob = qmm.qmm_packed_bytes(A, 16, 64)
    g = qmm.qmm_grouped_gemm
    expect(E_ARG, g, A, P, blob, 0, 16, 64, P, 4, P, P, P, 1, 4, 4, P, None, 0)      # n_experts
    expect(E_ARG, g, A, P, blob - 256, 2, 16, 64, P, 4, P, P, P, 1, 4, 4, P, None, 0)  # stride < blob
    expect(E_ARG, g, A, P, blob + 8, 2, 16, 64, P, 4, P, P, P, 1, 4, 4, P, None, 0)    # stride % 256
    expect(E_ARG, g, A, P, blob, 2, 16, 64, P, 4, P, None, P, 1, 4, 4, P, None, 0)     # NULL seg_expert
    expect(E_ARG, g, A, P, blob, 2, 16, 64, P, 4, P, P, P, 1, 4, 0, P, None, 0)        # max_seg_rows
    expect(E_ARG, g, A, P, blob, 2, 16, 64, P, 0, P, P, P, 1, 4, 4, P, None, 0)        # t_x
    expect(E_SHAPE, g, A, P, blob, 2, 16, 64, P, 4, P, P, P, 70000, 4, 4, P, None, 0)  # n_seg
    expect(E_ALIGN, g, A, P, blob, 2, 16, 64, P, 4, P + 2, P, P, 1, 4, 4, P, None, 0)
    assert "aligned" in qmm.qmm_last_error()
    ro = qmm.qmm_route
    expect(E_ARG, ro, None, 4, 64, P, 8, None, 2, P, P, P, P, P, 0)         # NULL x
    expect(E_ARG, ro, P, 0, 64, P, 8, None, 2, P, P, P, P, P, 0)            # t = 0
    expect(E_SHAPE, ro, P, 4, 64, P, 1025, None, 2, P, P, P, P, P, 0)       # too many experts
    expect(E_SHAPE, ro, P, 4, 64, P, 8, None, 9, P, P, P, P, P, 0)          # k > n_experts
    expect(E_SHAPE, ro, P, 4, 60, P, 8, None, 2, P, P, P, P, P, 0)          # d % 8
    expect(E_SHAPE, ro, P, 1 << 24, 8, P, 64, None, 64, P, P, P, P, P, 0)   # t*k = 2^30
    expect(E_ALIGN, ro, P + 8, 4, 64, P, 8, None, 2, P, P, P, P, P, 0)      # x 16-byte
    expect(E_ALIGN, ro, P, 4, 64, P, 8, P + 2, 2, P, P, P, P, P, 0)         # bias 4-byte
    gs = qmm.qmm_grouped_gemm_swiglu
    expect(E_SHAPE, gs, A, P, blob, 2, 15, 64, P, 4, P, P, P, 1, 4, 4, P, None, 0)      # odd n
    expect(E_ARG, gs, A, P, blob, 2, 16, 64, P, 4, P, None, P, 1, 4, 4, P, None, 0)     # NULL table
    g8 = qmm.qmm_gemv_int8
    expect(E_UNSUPPORTED, g8, M, P, 16, 64, P, P, 0)            # MXFP4
    expect(E_SHAPE, g8, A, P, 16, 57408, P, P, 0)               # d > 57344
    expect(E_ARG, g8, A, None, 16, 64, P, P, 0)                 # NULL packed
    expect(E_ALIGN, g8, A, P, 16, 64, P + 8, P, 0)              # x 16-byte
    expect(E_SHAPE, qmm.qmm_gemv, A, P, 1 << 27, 65536, P, P, None, 0)   # n*d/2 >= 2^31
    c = qmm.qmm_moe_combine
    expect(E_ARG, c, None, 8, 64, 4, 2, P, P, 8, P, P, P, 0)      # NULL o
    expect(E_SHAPE, c, P, 8, 64, 4, 65, P, P, 8, P, P, P, 0)      # k > 64
    expect(E_SHAPE, c, P, 8, 60, 4, 2, P, P, 8, P, P, P, 0)       # d % 8
    expect(E_ALIGN, c, P + 8, 8, 64, 4, 2, P, P, 8, P, P, P, 0)   # o 16-byte
    expect(E_ARG, c, P, 8, 64, 0, 2, P, P, 8, P, P, P, 0)         # t = 0
    s = qmm.qmm_stream_read
    expect(E_ARG, s, None, 1024, P, 0)
    expect(E_ARG, s, P, 1024, None, 0)
    expect(E_ALIGN, s, P + 8, 1024, P, 0)
    expect(E_SHAPE, s, P, 0, P, 0)
    expect(E_SHAPE, s, P, 1000, P, 0)
    expect(E_SHAPE, s, P, 1 << 31, P, 0)


def test_empty_grouped_call_is_a_no_op():
    blob = qmm.qmm_packed_bytes(A, 16, 64)
    qmm.qmm_grouped_gemm(A, P, blob, 2, 16, 64, P, 4, P, P, P, 0, 0, 1, P)   # n_seg = 0: returns OK


def test_product_path_has_no_fallback():
    import inspect
    src = inspect.getsource(qmm)
    assert "oracle" not in src and "numpy" not in src
