"""ctypes binding of libbwprobe.so: plain streaming kernels (read, copy, in-place
read-modify-write) in the replay kernels' access pattern, 32 KiB contiguous per work-group with
16-byte non-temporal accesses. The benchmark times them as the bandwidth ceilings that its
fractions of 8 TB/s are read against."""
import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbwprobe.so")
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: run __graft_entry__.build() first")
        L = ctypes.CDLL(_LIB_PATH)
        L.bwprobe_chunk_bytes.restype = ctypes.c_size_t
        L.bwprobe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
        L.bwprobe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        L.bwprobe_rmw.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_float, ctypes.c_void_p]
        for f in (L.bwprobe_read, L.bwprobe_copy, L.bwprobe_rmw):
            f.restype = ctypes.c_int
        _lib = L
    return _lib


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"{what} failed ({rc})")


def read(src: torch.Tensor, sink: torch.Tensor):
    """Read all of src (float32, a multiple of 32 KiB); sink: float32 of src.numel() // 2048."""
    assert src.dtype == torch.float32 and src.is_contiguous() and sink.dtype == torch.float32
    assert sink.numel() >= src.numel() * 4 // 8192
    _check(lib().bwprobe_read(src.data_ptr(), src.numel() * 4, sink.data_ptr(), _stream()), "bwprobe_read")


def copy(src: torch.Tensor, dst: torch.Tensor):
    assert src.dtype == dst.dtype == torch.float32 and src.numel() == dst.numel()
    assert src.is_contiguous() and dst.is_contiguous()
    _check(lib().bwprobe_copy(src.data_ptr(), dst.data_ptr(), src.numel() * 4, _stream()), "bwprobe_copy")


def rmw(buf: torch.Tensor, scale: float):
    assert buf.dtype == torch.float32 and buf.is_contiguous()
    _check(lib().bwprobe_rmw(buf.data_ptr(), buf.numel() * 4, float(scale), _stream()), "bwprobe_rmw")
