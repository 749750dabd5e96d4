"""Binding of libwkv7_probe (ctypes): the hardware-ceiling probes that
measurement code reads roofline fractions against — a streaming copy and a
matrix-core loop. Not part of the WKV-7 library; argument marshalling only.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libwkv7_probe.so")

EXPORTS = ("hwprobe_copy", "hwprobe_mfma", "hwprobe_mfma_per_iter")

MFMA_BF16 = 0      # v_mfma_f32_16x16x32_bf16: 16,384 flops per instruction
MFMA_I8 = 1        # v_mfma_i32_16x16x64_i8: 32,768 ops per instruction
MFMA_I8_32 = 2     # v_mfma_i32_32x32x32_i8: 65,536 ops per instruction
OPS_PER_MFMA = {MFMA_BF16: 2 * 16 * 16 * 32, MFMA_I8: 2 * 16 * 16 * 64,
                MFMA_I8_32: 2 * 32 * 32 * 32}
WAVES_PER_BLOCK = 4


class ProbeError(RuntimeError):
    pass


def _load() -> ctypes.CDLL:
    import torch  # noqa: F401  (bind to torch's HIP runtime)
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built "
                          "(python -m linear_attention_rnn_amd.build)")
    lib = ctypes.CDLL(LIB_PATH)
    lib.hwprobe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p,
                                 ctypes.c_size_t, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_void_p]
    lib.hwprobe_copy.restype = ctypes.c_int
    lib.hwprobe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_void_p, ctypes.c_size_t,
                                 ctypes.c_void_p]
    lib.hwprobe_mfma.restype = ctypes.c_int
    lib.hwprobe_mfma_per_iter.argtypes = []
    lib.hwprobe_mfma_per_iter.restype = ctypes.c_int
    return lib


lib = _load()


def _stream(stream) -> int:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream) or 0


def hwprobe_copy(src, dst, nbytes: int, nontemporal: bool = False,
                 blocks: int = 0, stream=None) -> None:
    """Copy `nbytes` from tensor `src` to tensor `dst` (the same tensor for
    an in-place pass) with the probe's uint4 stream kernel."""
    for t in (src, dst):
        if not t.is_cuda or not t.is_contiguous():
            raise ProbeError("src and dst must be contiguous device tensors")
        if t.numel() * t.element_size() < nbytes:
            raise ProbeError("buffer smaller than the copy")
    rc = lib.hwprobe_copy(src.data_ptr(), dst.data_ptr(), nbytes,
                          1 if nontemporal else 0, blocks, _stream(stream))
    if rc != 0:
        raise ProbeError(f"hwprobe_copy: hipError {rc}")


def hwprobe_mfma(kind: int, blocks: int, iters: int, out, stream=None) -> int:
    """Run the matrix-core loop; returns the ops it issues."""
    if not out.is_cuda or out.dtype.itemsize != 4 or not out.is_contiguous():
        raise ProbeError("out must be a contiguous 4-byte device tensor")
    rc = lib.hwprobe_mfma(kind, blocks, iters, out.data_ptr(), out.numel(),
                          _stream(stream))
    if rc != 0:
        raise ProbeError(f"hwprobe_mfma: hipError {rc}")
    return (blocks * WAVES_PER_BLOCK * iters * lib.hwprobe_mfma_per_iter()
            * OPS_PER_MFMA[kind])
