"""ctypes binding of libwanpeak.so (include/wanpeak.h): the sustained bf16
MFMA loop and the streaming device copy, read and write that the benchmark
quotes the library's kernels against, next to the spec peaks. Argument marshalling
only; not part of the attention path."""

from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libwanpeak.so")
THREADS = 256                      # WANPEAK_MFMA_THREADS
STREAM_BLOCK_BYTES = 16384         # WANPEAK_STREAM_BLOCK_BYTES
FLOP_PER_MFMA = 2 * 32 * 32 * 16   # v_mfma_f32_32x32x16_bf16

_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built (python __graft_entry__.py build)")
        L = ctypes.CDLL(LIB_PATH)
        L.wanpeak_mfma_bf16_loop.restype = ctypes.c_int
        L.wanpeak_mfma_bf16_loop.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                             ctypes.c_int, ctypes.c_void_p]
        L.wanpeak_copy.restype = ctypes.c_int
        L.wanpeak_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                   ctypes.c_void_p]
        L.wanpeak_read.restype = ctypes.c_int
        L.wanpeak_read.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                   ctypes.c_void_p]
        L.wanpeak_fill.restype = ctypes.c_int
        L.wanpeak_fill.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_uint32,
                                   ctypes.c_void_p]
        _lib = L
    return _lib


def mfma_loop_flop(blocks: int, iters: int) -> float:
    """FLOP of one wanpeak_mfma_bf16_loop launch (4 waves x 4 MFMAs per iteration)."""
    return float(blocks) * (THREADS // 64) * iters * 4 * FLOP_PER_MFMA


def mfma_bf16_loop(operands: torch.Tensor, out: torch.Tensor, blocks: int, iters: int) -> None:
    """operands: bf16 [2 * THREADS * 8] on the GPU; out: fp32 [blocks * THREADS]."""
    if operands.dtype != torch.bfloat16 or operands.numel() != 2 * THREADS * 8 or \
            not operands.is_contiguous() or not operands.is_cuda:
        raise ValueError("operands must be a contiguous bf16 CUDA tensor of 4096 elements")
    if out.dtype != torch.float32 or out.numel() != blocks * THREADS or not out.is_cuda:
        raise ValueError("out must be a float32 CUDA tensor of blocks * 256 elements")
    st = lib().wanpeak_mfma_bf16_loop(operands.data_ptr(), out.data_ptr(), blocks, iters,
                                      torch.cuda.current_stream(operands.device).cuda_stream)
    if st:
        raise RuntimeError(f"wanpeak_mfma_bf16_loop returned {st}")


def copy(dst: torch.Tensor, src: torch.Tensor) -> None:
    """dst[:] = src[:] for two contiguous CUDA tensors of the same byte size."""
    n = src.numel() * src.element_size()
    if not (src.is_cuda and dst.is_cuda and src.is_contiguous() and dst.is_contiguous()) or \
            dst.numel() * dst.element_size() != n:
        raise ValueError("src and dst must be contiguous CUDA tensors of the same size")
    st = lib().wanpeak_copy(dst.data_ptr(), src.data_ptr(), n,
                            torch.cuda.current_stream(src.device).cuda_stream)
    if st:
        raise RuntimeError(f"wanpeak_copy returned {st}")


def read_blocks(nbytes: int) -> int:
    """Words of `out` that read() needs for a source of nbytes."""
    return (nbytes + STREAM_BLOCK_BYTES - 1) // STREAM_BLOCK_BYTES


def read(out: torch.Tensor, src: torch.Tensor) -> None:
    """Reads every byte of src (contiguous CUDA tensor); out (int32 CUDA tensor of
    read_blocks(bytes) elements) receives each 16 KiB block's XOR of 4-byte words."""
    n = src.numel() * src.element_size()
    if not (src.is_cuda and src.is_contiguous()) or n % 16:
        raise ValueError("src must be a contiguous CUDA tensor of a multiple of 16 bytes")
    if out.dtype != torch.int32 or out.numel() != read_blocks(n) or not out.is_cuda or \
            not out.is_contiguous():
        raise ValueError("out must be a contiguous int32 CUDA tensor of read_blocks(bytes) elements")
    st = lib().wanpeak_read(out.data_ptr(), src.data_ptr(), n,
                            torch.cuda.current_stream(src.device).cuda_stream)
    if st:
        raise RuntimeError(f"wanpeak_read returned {st}")


def fill(dst: torch.Tensor, value: int) -> None:
    """Sets every 4-byte word of dst (contiguous CUDA tensor) to value."""
    n = dst.numel() * dst.element_size()
    if not (dst.is_cuda and dst.is_contiguous()) or n % 16:
        raise ValueError("dst must be a contiguous CUDA tensor of a multiple of 16 bytes")
    st = lib().wanpeak_fill(dst.data_ptr(), n, value & 0xFFFFFFFF,
                            torch.cuda.current_stream(dst.device).cuda_stream)
    if st:
        raise RuntimeError(f"wanpeak_fill returned {st}")
