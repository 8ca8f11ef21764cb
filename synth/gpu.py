"""Device-side fill of the generator's integer streams (libsynth.so).

Bit-identical to ``synth.code_bytes`` / ``synth.small_int``; used to build the
routed-expert weight stacks directly in device memory.
"""
from __future__ import annotations

import ctypes
import os

import synth

_lib = None


def load():
    global _lib
    if _lib is None:
        import torch  # noqa: F401  (torch's HIP runtime is the process's; see bit_weight_quantized_amd.load)
        path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsynth.so")
        if not os.path.exists(path):
            raise ImportError(f"{path} is missing: build with `python -m bit_weight_quantized_amd.build`")
        lib = ctypes.CDLL(path)
        u32, i64, vp = ctypes.c_uint32, ctypes.c_int64, ctypes.c_void_p
        lib.synth_key.restype = ctypes.c_uint64
        lib.synth_key.argtypes = [u32, u32, u32]
        lib.synth_code_bytes.restype = ctypes.c_int
        lib.synth_code_bytes.argtypes = [u32, u32, u32, vp, i64, i64, vp]
        lib.synth_small_int_u8.restype = ctypes.c_int
        lib.synth_small_int_u8.argtypes = [u32, u32, u32, vp, i64, i64, u32, u32, vp]
        _lib = lib
    return _lib


def _stream():
    import torch
    return torch.cuda.current_stream().cuda_stream


def code_bytes(seed: int, stream: int, sub: int, dst, start_byte: int = 0) -> None:
    """Fill the uint8 tensor `dst` with hash-stream bytes [start_byte, start_byte + numel)."""
    err = load().synth_code_bytes(seed, stream, sub, dst.data_ptr(), dst.numel() * dst.element_size(),
                                  start_byte, _stream())
    if err:
        raise RuntimeError(f"synth_code_bytes: hipError {err}")


def small_int_u8(seed: int, stream: int, sub: int, dst, lo: int, m: int, start: int = 0) -> None:
    err = load().synth_small_int_u8(seed, stream, sub, dst.data_ptr(), dst.numel(), start, lo, m,
                                    _stream())
    if err:
        raise RuntimeError(f"synth_small_int_u8: hipError {err}")


def expert_stack(seed: int, which: str, n_experts: int, pack, packed_bytes: int, stride: int,
                 out, device="cuda"):
    """Generate every expert's canonical MXFP4 weights on the device and pack
    each into `out` (uint8, n_experts * stride bytes) with `pack(codes, e8m0,
    dst_ptr)`.  `which` is "gate_up" or "down"."""
    import torch
    n, d, cs, es = {"gate_up": (6144, 3584, synth.S_GU_CODES, synth.S_GU_E8M0),
                    "down": (3584, 3072, synth.S_DN_CODES, synth.S_DN_E8M0)}[which]
    codes = torch.empty(n * d // 2, dtype=torch.uint8, device=device)
    e8m0 = torch.empty(n * d // 32, dtype=torch.uint8, device=device)
    base = out.data_ptr()
    for e in range(n_experts):
        code_bytes(seed, cs, e, codes)
        small_int_u8(seed, es, e, e8m0, 118, 9)
        pack(codes, e8m0, base + e * stride)
    return n, d
