"""Python binding of libyoco_ceiling.so (achievable-rate probes): argument
marshalling only, like the binding of libyoco.so. The probes are plain
streaming kernels with the traffic pattern of the decode (one read of a buffer)
and of the compose (four reads, two writes), and back-to-back bf16 MFMAs on
caller-supplied operands for the prefill, with none of the method's
arithmetic; the benchmark times them beside the kernels they bound."""
from __future__ import annotations

import ctypes
import os

import torch

from .binding import YocoError, _stream

_HERE = os.path.dirname(os.path.abspath(__file__))
CEILING_LIB_PATH = os.path.join(_HERE, "libyoco_ceiling.so")
CEILING_EXPORTED = ("yoco_ceiling_read", "yoco_ceiling_read_blocks", "yoco_ceiling_read4_write2",
                    "yoco_ceiling_mfma_bf16", "yoco_ceiling_last_error")

_lib = None


def load_ceiling_library(path: str = CEILING_LIB_PATH) -> ctypes.CDLL:
    """Load libyoco_ceiling.so once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m cross_layer_shared_amd.build`")
    lib = ctypes.CDLL(path)
    i, vp, sz = ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
    lib.yoco_ceiling_read.argtypes = [vp, sz, i, i, i, i, vp, vp]
    lib.yoco_ceiling_read.restype = i
    lib.yoco_ceiling_read_blocks.argtypes = [vp, sz, i, i, i, vp, vp]
    lib.yoco_ceiling_read_blocks.restype = i
    lib.yoco_ceiling_read4_write2.argtypes = [vp, vp, vp, vp, vp, vp, sz, i, i, vp]
    lib.yoco_ceiling_read4_write2.restype = i
    lib.yoco_ceiling_mfma_bf16.argtypes = [vp, sz, i, i, vp, vp]
    lib.yoco_ceiling_mfma_bf16.restype = i
    lib.yoco_ceiling_last_error.argtypes = []
    lib.yoco_ceiling_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != 0:
        raise YocoError(status, load_ceiling_library().yoco_ceiling_last_error().decode())


def _nbytes(t: torch.Tensor) -> int:
    if not t.is_contiguous():
        raise ValueError("probe buffers must be contiguous")
    return t.numel() * t.element_size()


def yoco_ceiling_read(src: torch.Tensor, sink: torch.Tensor, workgroups: int = 256, threads: int = 512,
                      loads_per_thread: int = 8, nontemporal: bool = True, stream=None) -> None:
    """Read every byte of src once (see yoco_ceiling.h); sink is a device int32/uint32 [>= 1]."""
    _check(load_ceiling_library().yoco_ceiling_read(src.data_ptr(), _nbytes(src), int(workgroups), int(threads),
                                                    int(loads_per_thread), int(bool(nontemporal)), sink.data_ptr(),
                                                    _stream(stream)))


def yoco_ceiling_read_blocks(src: torch.Tensor, sink: torch.Tensor, workgroups: int = 256, threads: int = 512,
                             loads_per_thread: int = 8, stream=None) -> None:
    """Read every byte of src once, each wavefront in contiguous blocks (see yoco_ceiling.h)."""
    _check(load_ceiling_library().yoco_ceiling_read_blocks(src.data_ptr(), _nbytes(src), int(workgroups), int(threads),
                                                           int(loads_per_thread), sink.data_ptr(), _stream(stream)))


def yoco_ceiling_read4_write2(a, b, c, d, e, f, threads: int = 512, positions_per_thread: int = 1,
                              stream=None) -> None:
    """e = a + b, f = c + d as 32-bit integers; six equally sized contiguous buffers."""
    n = _nbytes(a)
    for t in (b, c, d, e, f):
        if _nbytes(t) != n:
            raise ValueError("the six buffers must have the same size")
    _check(load_ceiling_library().yoco_ceiling_read4_write2(a.data_ptr(), b.data_ptr(), c.data_ptr(), d.data_ptr(),
                                                            e.data_ptr(), f.data_ptr(), n, int(threads),
                                                            int(positions_per_thread), _stream(stream)))


MFMA_THREADS = 512
MFMA_FLOP = 32 * 32 * 16 * 2      # one v_mfma_f32_32x32x16_bf16


def mfma_flop(workgroups: int, iters: int) -> float:
    """Floating-point operations of one yoco_ceiling_mfma_bf16 call."""
    return float(workgroups) * (MFMA_THREADS // 64) * iters * 16 * MFMA_FLOP


def yoco_ceiling_mfma_bf16(operands: torch.Tensor, sink: torch.Tensor, workgroups: int = 256, iters: int = 4096,
                           stream=None) -> None:
    """Back-to-back bf16 MFMAs on operands from the bf16 pool `operands`; sink is a device float32 [>= 1]."""
    if operands.dtype != torch.bfloat16:
        raise ValueError("operands must be bfloat16")
    _check(load_ceiling_library().yoco_ceiling_mfma_bf16(operands.data_ptr(), _nbytes(operands), int(workgroups),
                                                         int(iters), sink.data_ptr(), _stream(stream)))
