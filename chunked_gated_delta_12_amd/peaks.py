"""Binding of libkda_peaks (include/kda_peaks.h): the on-device reference
measurements the benchmark sets its rates against.  Argument marshalling only;
the work runs in the library's HIP kernels."""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkda_peaks.so")
HEADER_PATH = os.path.join(_HERE, "..", "include", "kda_peaks.h")
MFMA_FLOP = 16 * 16 * 32 * 2   # one v_mfma_f32_16x16x32_bf16
_lib = None


class DeviceInfo(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 256), ("arch", ctypes.c_char * 64),
                ("compute_units", ctypes.c_int), ("clock_khz", ctypes.c_int),
                ("memory_clock_khz", ctypes.c_int), ("memory_bus_bits", ctypes.c_int),
                ("l2_bytes", ctypes.c_int), ("total_bytes", ctypes.c_longlong),
                ("lds_bytes_per_cu", ctypes.c_int), ("warp_size", ctypes.c_int)]


def load_library(path: str = LIB_PATH):
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise RuntimeError(f"{path} not found: build it first (python -m chunked_gated_delta_12_amd.build)")
        lib = ctypes.CDLL(path)
        lib.kda_peaks_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        lib.kda_peaks_copy.restype = ctypes.c_int
        lib.kda_peaks_mfma_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        lib.kda_peaks_mfma_bf16.restype = ctypes.c_int
        lib.kda_peaks_device.argtypes = [ctypes.c_int, ctypes.POINTER(DeviceInfo)]
        lib.kda_peaks_device.restype = ctypes.c_int
        _lib = lib
    return _lib


def _stream(stream, dev):
    return ctypes.c_void_p((stream or torch.cuda.current_stream(dev)).cuda_stream)


def copy(src: torch.Tensor, dst: torch.Tensor, stream=None) -> None:
    """dst <- src, bytewise, with the library's streaming copy kernel."""
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != n or not (src.is_contiguous() and dst.is_contiguous()):
        raise ValueError("src and dst must be contiguous and of the same byte size")
    st = load_library().kda_peaks_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), n,
                                       _stream(stream, src.device))
    if st:
        raise RuntimeError(f"kda_peaks_copy failed ({st})")


def mfma_bf16(sink: torch.Tensor, workgroups: int, iters: int, stream=None) -> int:
    """Runs the bf16 matrix-core loop; returns the flop it performs."""
    if sink.dtype != torch.float32 or sink.numel() < workgroups * 256:
        raise ValueError("sink must be a float32 tensor of at least workgroups*256 elements")
    st = load_library().kda_peaks_mfma_bf16(ctypes.c_void_p(sink.data_ptr()), workgroups, iters,
                                            _stream(stream, sink.device))
    if st:
        raise RuntimeError(f"kda_peaks_mfma_bf16 failed ({st})")
    return workgroups * 4 * iters * 8 * MFMA_FLOP


def device_info(device: int = 0) -> dict:
    info = DeviceInfo()
    st = load_library().kda_peaks_device(device, ctypes.byref(info))
    if st:
        raise RuntimeError(f"kda_peaks_device failed ({st})")
    return {"name": info.name.decode(), "arch": info.arch.decode(), "compute_units": info.compute_units,
            "clock_mhz": info.clock_khz / 1e3, "memory_clock_mhz": info.memory_clock_khz / 1e3,
            "memory_bus_bits": info.memory_bus_bits, "l2_bytes": info.l2_bytes,
            "total_bytes": info.total_bytes, "lds_bytes_per_cu": info.lds_bytes_per_cu,
            "warp_size": info.warp_size}
