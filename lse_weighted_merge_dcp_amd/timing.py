"""HIP events for timing single libdcpmerge calls (dcp_time_next_call).

The events come from the HIP runtime this process already runs (torch and
libdcpmerge share it) and are created with hipEventDisableSystemFence, so
that attaching them to a kernel dispatch adds no system-scope cache release
to the kernel being timed.  Measurement plumbing only: nothing here touches
the merge's data.
"""
from __future__ import annotations

import ctypes

from . import _lib

HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000

_hip = None


def hip_runtime():
    """The libamdhip64 mapped into this process (loaded by libdcpmerge's
    dependencies if nothing loaded it before)."""
    global _hip
    if _hip is None:
        _lib.lib()
        path = None
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64.so" in line:
                    path = line.split()[-1]
                    break
        if path is None:
            raise RuntimeError("the HIP runtime is not loaded in this process")
        h = ctypes.CDLL(path)
        h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        h.hipEventDestroy.argtypes = [ctypes.c_void_p]
        h.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        for fn in (h.hipEventCreateWithFlags, h.hipEventDestroy, h.hipEventSynchronize, h.hipEventElapsedTime,
                   h.hipGetLastError):
            fn.restype = ctypes.c_int
        _hip = h
    return _hip


def _ok(rc: int, what: str) -> None:
    if rc != 0:
        # the failed call also left its code as the thread's last HIP error,
        # which the next unrelated HIP user (torch) would report as its own
        hip_runtime().hipGetLastError()
        raise RuntimeError("%s failed with hipError_t %d" % (what, rc))


class Event:
    """A HIP timing event on the current device."""

    def __init__(self):
        self._h = ctypes.c_void_p()
        self._rt = hip_runtime()
        _ok(self._rt.hipEventCreateWithFlags(ctypes.byref(self._h), HIP_EVENT_DISABLE_SYSTEM_FENCE),
            "hipEventCreateWithFlags")

    @property
    def handle(self) -> int:
        return self._h.value

    def synchronize(self) -> None:
        _ok(self._rt.hipEventSynchronize(self._h), "hipEventSynchronize")

    def elapsed_us(self, later: "Event") -> float:
        """Microseconds from this event to `later` (both recorded)."""
        ms = ctypes.c_float()
        _ok(self._rt.hipEventElapsedTime(ctypes.byref(ms), self._h, later._h), "hipEventElapsedTime")
        return ms.value * 1e3

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            self._rt.hipEventDestroy(h)
            self._h = None
