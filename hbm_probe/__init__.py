"""hbm_probe -- the HBM read-ceiling probe that bench.py reports beside the
statistics kernel's roofline: a ctypes binding of libvpa_probe.so
(hbm_probe/vpa_probe.h, built from hbm_probe/read_probe.hip by
hbm_probe/build.py).  Measurement only: the argmax library neither contains
nor calls it, and only bench.py and tests/test_read_probe.py load it.
hbm_probe/block_sizes.py is a separate program for hardware-counter runs:
it launches the library's statistics kernel with two block sizes."""
import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libvpa_probe.so")
SYMBOLS = ("vpa_probe_read_bytes", "vpa_probe_sink_words", "vpa_probe_read")
WORKGROUPS_PER_CU = 2      # the fastest residency measured on MI355X

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m vocab_argmax_amd._build` (hipcc, gfx950)")
        lb = ctypes.CDLL(LIB_PATH)
        lb.vpa_probe_read_bytes.argtypes = [ctypes.c_int64]
        lb.vpa_probe_read_bytes.restype = ctypes.c_int64
        lb.vpa_probe_sink_words.argtypes = [ctypes.c_int32]
        lb.vpa_probe_sink_words.restype = ctypes.c_int64
        lb.vpa_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                      ctypes.c_int32, ctypes.c_void_p]
        lb.vpa_probe_read.restype = ctypes.c_int
        _lib = lb
    return _lib


def default_workgroups(device) -> int:
    return WORKGROUPS_PER_CU * torch.cuda.get_device_properties(device).multi_processor_count


def make_sink(device, n_workgroups):
    return torch.empty(lib().vpa_probe_sink_words(n_workgroups), dtype=torch.int32, device=device)


def read(buf, sink, n_workgroups):
    """Enqueue one read of `buf` (a contiguous device tensor) on the current
    stream of its device; returns the bytes read (whole 4 KiB chunks)."""
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    if sink.device != buf.device or sink.dtype != torch.int32 or not sink.is_contiguous():
        raise ValueError("sink must be a contiguous int32 tensor on the buffer's device")
    if sink.numel() < lib().vpa_probe_sink_words(n_workgroups):
        raise ValueError("sink is smaller than vpa_probe_sink_words(n_workgroups)")
    nbytes = buf.numel() * buf.element_size()
    stream = torch.cuda.current_stream(buf.device).cuda_stream
    with torch.cuda.device(buf.device):
        rc = lib().vpa_probe_read(ctypes.c_void_p(buf.data_ptr()), nbytes,
                                  ctypes.c_void_p(sink.data_ptr()), n_workgroups,
                                  ctypes.c_void_p(stream))
    if rc != 0:
        raise RuntimeError(f"vpa_probe_read failed ({rc})")
    return lib().vpa_probe_read_bytes(nbytes)
