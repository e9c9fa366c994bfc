"""Minimal ctypes access to HIP events in libamdhip64 (timing plumbing)."""
from __future__ import annotations

import ctypes
import ctypes.util
import os

_hip = None


def _load():
    global _hip
    if _hip is None:
        for cand in ("/opt/rocm/lib/libamdhip64.so", ctypes.util.find_library("amdhip64"),
                     "libamdhip64.so"):
            if cand and (os.path.exists(cand) or not cand.startswith("/")):
                try:
                    _hip = ctypes.CDLL(cand)
                    break
                except OSError:
                    continue
        if _hip is None:
            raise OSError("libamdhip64.so not found")
        _hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        _hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        _hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        _hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        _hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                             ctypes.c_void_p]
    return _hip


def _ok(rc, what):
    if rc != 0:
        raise RuntimeError(f"{what} failed with HIP error {rc}")


class Event:
    """A HIP event (timing enabled)."""

    def __init__(self):
        self.handle = ctypes.c_void_p()
        _ok(_load().hipEventCreate(ctypes.byref(self.handle)), "hipEventCreate")

    @property
    def ptr(self):
        return self.handle.value

    def record(self, stream_handle: int):
        _ok(_load().hipEventRecord(self.handle, ctypes.c_void_p(stream_handle)), "hipEventRecord")

    def synchronize(self):
        _ok(_load().hipEventSynchronize(self.handle), "hipEventSynchronize")

    def elapsed_ms(self, end: "Event") -> float:
        ms = ctypes.c_float()
        _ok(_load().hipEventElapsedTime(ctypes.byref(ms), self.handle, end.handle),
            "hipEventElapsedTime")
        return float(ms.value)

    def __del__(self):
        try:
            if self.handle and _hip is not None:
                _hip.hipEventDestroy(self.handle)
        except Exception:
            pass
