"""Python binding of libqmm, the MI355X 4-bit weight-quantized matmul library.

Argument marshalling only: every function here forwards to the C ABI of the
same name in ``libqmm.so`` (declared in ``include/qmm.h``); all computation
runs in the library's HIP kernels.  Pointer arguments accept a torch tensor
(its ``data_ptr()``), a raw integer address, or ``None`` for NULL.  Calls are
asynchronous on ``stream`` (default: torch's current stream).  A non-OK status
raises :class:`QmmError`; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "QMM_AFFINE4_G64", "QMM_MXFP4_G32", "QmmError", "lib_path", "load",
    "qmm_packed_bytes", "qmm_workspace_bytes", "qmm_pack", "qmm_unpack", "qmm_gemv",
    "qmm_gemm", "qmm_grouped_gemm", "qmm_status_string", "qmm_last_error",
    "qmm_layout_version", "qmm_profile_next", "qmm_stream_read", "qmm_route",
    "qmm_grouped_gemm_swiglu", "qmm_moe_combine", "qmm_gemv_int8", "qmm_gemm_noalloc", "qmm_set_kernel", "qmm_get_kernel",
    "QMM_KERNEL_AUTO", "QMM_KERNEL_TILE", "QMM_KERNEL_TILE_UNSPLIT", "QMM_KERNEL_FEW_ROW",
    "QMM_KERNEL_GROUPED_MATMUL", "QMM_KERNEL_MULTI_ROW", "EXPORTS",
]

QMM_AFFINE4_G64 = 1
QMM_MXFP4_G32 = 2

QMM_KERNEL_AUTO = 0
QMM_KERNEL_TILE = 1
QMM_KERNEL_TILE_UNSPLIT = 2
QMM_KERNEL_FEW_ROW = 3
QMM_KERNEL_GROUPED_MATMUL = 4
QMM_KERNEL_MULTI_ROW = 5

STATUS = {0: "QMM_OK", 1: "QMM_E_ARG", 2: "QMM_E_SHAPE", 3: "QMM_E_ALIGN", 4: "QMM_E_UNSUPPORTED",
          5: "QMM_E_WORKSPACE", 6: "QMM_E_HIP", 7: "QMM_E_LAYOUT", 8: "QMM_E_VALUE"}

EXPORTS = ("qmm_packed_bytes", "qmm_workspace_bytes", "qmm_pack", "qmm_unpack", "qmm_gemv",
           "qmm_gemm", "qmm_grouped_gemm", "qmm_status_string", "qmm_last_error",
           "qmm_layout_version", "qmm_profile_next", "qmm_stream_read", "qmm_route",
           "qmm_grouped_gemm_swiglu", "qmm_moe_combine", "qmm_gemv_int8", "qmm_gemm_noalloc",
           "qmm_set_kernel", "qmm_get_kernel")

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None


def lib_path() -> str:
    return os.path.join(_HERE, "libqmm.so")


class QmmError(RuntimeError):
    def __init__(self, status: int, func: str, detail: str):
        self.status = status
        self.name = STATUS.get(status, str(status))
        super().__init__(f"{func} -> {self.name}: {detail}")


def load():
    """Load libqmm.so (once).  Fails loudly when the library is not built."""
    global _lib
    if _lib is not None:
        return _lib
    # torch first: it ships its own libamdhip64.so.7, and whichever copy of
    # that soname a process loads first is the one every library binds to.
    # Loaded after torch, libqmm shares torch's HIP runtime (its streams and
    # allocations); loaded before, it would pull in the system copy and leave
    # torch on a runtime it was not built against.
    import torch  # noqa: F401
    path = lib_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python -m bit_weight_quantized_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(path)
    i64, i32, sz, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p
    sig = {
        "qmm_packed_bytes": (sz, [ctypes.c_int, i64, i64]),
        "qmm_workspace_bytes": (sz, [ctypes.c_int, i64, i64, i64]),
        "qmm_pack": (ctypes.c_int, [ctypes.c_int, i64, i64, vp, vp, vp, vp, vp]),
        "qmm_unpack": (ctypes.c_int, [ctypes.c_int, i64, i64, vp, vp, vp, vp, vp]),
        "qmm_gemv": (ctypes.c_int, [ctypes.c_int, vp, i64, i64, vp, vp, vp, sz, vp]),
        "qmm_gemm": (ctypes.c_int, [ctypes.c_int, vp, i64, i64, i64, vp, vp, vp, sz, vp]),
        "qmm_grouped_gemm": (ctypes.c_int, [ctypes.c_int, vp, i64, i32, i64, i64, vp, i64, vp, vp,
                                            vp, i32, i32, i32, vp, vp, sz, vp]),
        "qmm_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "qmm_last_error": (ctypes.c_char_p, []),
        "qmm_layout_version": (ctypes.c_uint32, []),
        "qmm_profile_next": (ctypes.c_int, [vp, vp]),
        "qmm_stream_read": (ctypes.c_int, [vp, sz, vp, vp]),
        "qmm_route": (ctypes.c_int, [vp, i64, i64, vp, i32, vp, i32, vp, vp, vp, vp, vp, vp]),
        "qmm_grouped_gemm_swiglu": (ctypes.c_int, [ctypes.c_int, vp, i64, i32, i64, i64, vp, i64, vp, vp,
                                                   vp, i32, i32, i32, vp, vp, sz, vp]),
        "qmm_moe_combine": (ctypes.c_int, [vp, i32, i64, i64, i32, vp, vp, i32, vp, vp, vp, vp]),
        "qmm_gemv_int8": (ctypes.c_int, [ctypes.c_int, vp, i64, i64, vp, vp, vp]),
        "qmm_gemm_noalloc": (ctypes.c_int, [ctypes.c_int, vp, i64, i64, i64, vp, vp, vp]),
        "qmm_set_kernel": (ctypes.c_int, [ctypes.c_int]),
        "qmm_get_kernel": (ctypes.c_int, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _ptr(v):
    if v is None:
        return None
    if isinstance(v, int):
        return v
    return v.data_ptr()


def _nbytes(v):
    if v is None:
        return 0
    if isinstance(v, int):
        raise TypeError("pass the workspace as a tensor so its size is known")
    return v.numel() * v.element_size()


def _stream(s):
    if s is None:
        import torch
        if torch.cuda.is_available():
            return torch.cuda.current_stream().cuda_stream
        return None
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(status: int, func: str):
    if status != 0:
        lib = load()
        raise QmmError(status, func, (lib.qmm_last_error() or b"").decode())


def qmm_packed_bytes(fmt: int, n: int, d: int) -> int:
    return int(load().qmm_packed_bytes(fmt, n, d))


def qmm_workspace_bytes(fmt: int, t: int, n: int, d: int) -> int:
    return int(load().qmm_workspace_bytes(fmt, t, n, d))


def qmm_layout_version() -> int:
    return int(load().qmm_layout_version())


def qmm_status_string(status: int) -> str:
    return load().qmm_status_string(status).decode()


def qmm_last_error() -> str:
    return (load().qmm_last_error() or b"").decode()


def qmm_profile_next(start_event, stop_event):
    """Arm two raw hipEvent_t handles (ints) for the next matmul launch on this thread."""
    _check(load().qmm_profile_next(start_event, stop_event), "qmm_profile_next")


def qmm_stream_read(src, nbytes, sink, stream=None):
    """Read `nbytes` of device memory once (measurement of the HBM read ceiling)."""
    _check(load().qmm_stream_read(_ptr(src), nbytes, _ptr(sink), _stream(stream)), "qmm_stream_read")


def qmm_route(x, t, d, r, n_experts, bias, k, scores, topk, seg_expert, seg_offsets, row_index,
              stream=None):
    _check(load().qmm_route(_ptr(x), t, d, _ptr(r), n_experts, _ptr(bias), k, _ptr(scores), _ptr(topk),
                            _ptr(seg_expert), _ptr(seg_offsets), _ptr(row_index), _stream(stream)),
           "qmm_route")


def qmm_pack(fmt, n, d, codes, scales, biases, packed, stream=None):
    _check(load().qmm_pack(fmt, n, d, _ptr(codes), _ptr(scales), _ptr(biases), _ptr(packed),
                           _stream(stream)), "qmm_pack")


def qmm_unpack(fmt, n, d, packed, codes, scales, biases, stream=None):
    _check(load().qmm_unpack(fmt, n, d, _ptr(packed), _ptr(codes), _ptr(scales), _ptr(biases),
                             _stream(stream)), "qmm_unpack")


def qmm_gemv(fmt, packed, n, d, x, y, ws=None, stream=None):
    _check(load().qmm_gemv(fmt, _ptr(packed), n, d, _ptr(x), _ptr(y), _ptr(ws), _nbytes(ws),
                           _stream(stream)), "qmm_gemv")


def qmm_gemm(fmt, packed, t, n, d, x, y, ws=None, stream=None):
    _check(load().qmm_gemm(fmt, _ptr(packed), t, n, d, _ptr(x), _ptr(y), _ptr(ws), _nbytes(ws),
                           _stream(stream)), "qmm_gemm")


def qmm_gemm_noalloc(fmt, packed, t, n, d, x, y, stream=None):
    _check(load().qmm_gemm_noalloc(fmt, _ptr(packed), t, n, d, _ptr(x), _ptr(y), _stream(stream)),
           "qmm_gemm_noalloc")


def qmm_set_kernel(kernel):
    """Force one matmul kernel process-wide (QMM_KERNEL_*), or AUTO."""
    _check(load().qmm_set_kernel(kernel), "qmm_set_kernel")


def qmm_get_kernel():
    """The current kernel setting; -1 if QMM_FORCE_KERNEL holds an unknown value."""
    return load().qmm_get_kernel()


def qmm_grouped_gemm(fmt, packed_stack, expert_stride_bytes, n_experts, n, d, x, t_x, row_index,
                     seg_expert, seg_offsets, n_seg, m_total, max_seg_rows, y, ws=None,
                     stream=None):
    _check(load().qmm_grouped_gemm(fmt, _ptr(packed_stack), expert_stride_bytes, n_experts, n, d,
                                   _ptr(x), t_x, _ptr(row_index), _ptr(seg_expert),
                                   _ptr(seg_offsets), n_seg, m_total, max_seg_rows, _ptr(y),
                                   _ptr(ws), _nbytes(ws), _stream(stream)), "qmm_grouped_gemm")


def qmm_grouped_gemm_swiglu(fmt, packed_stack, expert_stride_bytes, n_experts, n, d, x, t_x, row_index,
                            seg_expert, seg_offsets, n_seg, m_total, max_seg_rows, h, ws=None,
                            stream=None):
    _check(load().qmm_grouped_gemm_swiglu(fmt, _ptr(packed_stack), expert_stride_bytes, n_experts, n, d,
                                          _ptr(x), t_x, _ptr(row_index), _ptr(seg_expert),
                                          _ptr(seg_offsets), n_seg, m_total, max_seg_rows, _ptr(h),
                                          _ptr(ws), _nbytes(ws), _stream(stream)), "qmm_grouped_gemm_swiglu")


def qmm_moe_combine(o, m_total, d, t, k, topk, weights, n_experts, seg_offsets, row_index, out,
                    stream=None):
    _check(load().qmm_moe_combine(_ptr(o), m_total, d, t, k, _ptr(topk), _ptr(weights), n_experts,
                                  _ptr(seg_offsets), _ptr(row_index), _ptr(out), _stream(stream)),
           "qmm_moe_combine")


def qmm_gemv_int8(fmt, packed, n, d, x, y, stream=None):
    _check(load().qmm_gemv_int8(fmt, _ptr(packed), n, d, _ptr(x), _ptr(y), _stream(stream)), "qmm_gemv_int8")
