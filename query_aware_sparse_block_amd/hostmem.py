"""Pinned host memory that kernels read directly, for a K/V pool kept in host
RAM (the setting of the SparPR page, where the full cache lives off the GPU
and only what is selected crosses to it).

The buffer comes from hipHostMalloc with the mapped flag, and the address the
kernels use comes from hipHostGetDevicePointer, so device access is what the
HIP API promises for it rather than an assumption about unified addressing.
The HIP runtime used is the one already loaded in the process (the one the
library's launches go through)."""

from __future__ import annotations

import ctypes

import numpy as np

_HIP_HOST_MALLOC_MAPPED = 0x2
_hip = None


def _runtime():
    global _hip
    if _hip is None:
        import torch  # noqa: F401  loads the process's HIP runtime first
        L = ctypes.CDLL("libamdhip64.so.7")
        L.hipHostMalloc.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t,
                                    ctypes.c_uint]
        L.hipHostMalloc.restype = ctypes.c_int
        L.hipHostGetDevicePointer.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p,
                                              ctypes.c_uint]
        L.hipHostGetDevicePointer.restype = ctypes.c_int
        L.hipHostFree.argtypes = [ctypes.c_void_p]
        L.hipHostFree.restype = ctypes.c_int
        _hip = L
    return _hip


class HostBuffer:
    """`nbytes` of mapped pinned host memory: `.array(dtype, shape)` views it
    from the host, `.device_ptr` is the address kernels use."""

    def __init__(self, nbytes: int):
        L = _runtime()
        self.nbytes = int(nbytes)
        self._host = ctypes.c_void_p()
        rc = L.hipHostMalloc(ctypes.byref(self._host), self.nbytes, _HIP_HOST_MALLOC_MAPPED)
        if rc != 0 or not self._host.value:
            raise RuntimeError(f"hipHostMalloc of {self.nbytes} bytes failed (error {rc})")
        dev = ctypes.c_void_p()
        rc = L.hipHostGetDevicePointer(ctypes.byref(dev), self._host, 0)
        if rc != 0 or not dev.value:
            L.hipHostFree(self._host)
            raise RuntimeError(f"hipHostGetDevicePointer failed (error {rc})")
        self.device_ptr = dev.value

    def array(self, dtype, shape) -> np.ndarray:
        n = int(np.prod(shape)) * np.dtype(dtype).itemsize
        assert n <= self.nbytes
        raw = (ctypes.c_uint8 * n).from_address(self._host.value)
        return np.frombuffer(raw, dtype=dtype).reshape(shape)

    def close(self):
        if self._host is not None and self._host.value:
            _runtime().hipHostFree(self._host)
        self._host = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def host_copy(arr: np.ndarray) -> HostBuffer:
    """A mapped pinned copy of a host array (16-bit payloads keep their bits)."""
    arr = np.ascontiguousarray(arr)
    buf = HostBuffer(arr.nbytes)
    buf.array(arr.dtype, arr.shape)[...] = arr
    return buf
