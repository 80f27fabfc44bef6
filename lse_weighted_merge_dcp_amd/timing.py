"""Device time of single libdcpmerge calls, for measurement only.

A timed call runs the same kernels through libdcpmerge_bench.so (built from
the same sources, csrc/dcpmerge_bench.h), whose dcpb_* calls take two HIP
events and attach them to the call's own kernel dispatches: the start event
records when the first kernel starts, the stop event when the last one ends.
libdcpmerge.so itself takes no events and keeps no state.  ops.py sends a
call here when it is given `timing=(start, stop)`.

The events come from the HIP runtime this process already runs (torch and
the libraries share it) and are created with hipEventDisableSystemFence, so
that attaching them to a kernel dispatch adds no system-scope cache release
to the kernel being timed.  Nothing here touches the merge's data.
"""
from __future__ import annotations

import ctypes
import os

from . import _lib

HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000
BENCH_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdcpmerge_bench.so")
DCPB_ERR_CAPTURE = -10
_bench = None


class CaptureError(_lib.DcpError):
    """A timed call was made on a stream that is being captured (nothing
    was enqueued): a capture does not keep dispatch events."""

    def __init__(self, fn: str):
        ValueError.__init__(self, "%s failed: DCPB_ERR_CAPTURE (timing events on a capturing stream)" % fn)
        self.status = DCPB_ERR_CAPTURE


def bench_lib():
    """libdcpmerge_bench.so, loaded on first use (raises if it is not built)."""
    global _bench
    if _bench is None:
        if not os.path.exists(BENCH_LIB_PATH):
            raise ImportError("libdcpmerge_bench.so is not built (expected at %s); run "
                              "`python -m lse_weighted_merge_dcp_amd.csrc.build`" % BENCH_LIB_PATH)
        h = ctypes.CDLL(BENCH_LIB_PATH)
        for name in ("dcp_pack", "dcp_unpack_combine", "dcp_lse_combine_inplace"):
            args, res = _lib.SIGNATURES[name]
            fn = getattr(h, "dcpb_" + name[len("dcp_"):])
            fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p] + list(args) + [ctypes.c_void_p]
            fn.restype = res
        h.dcpb_empty_kernel.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
        h.dcpb_empty_kernel.restype = ctypes.c_int
        _bench = h
    return _bench


class LaunchShape:
    """What a call launched: launches, workgroups of its last launch and
    threads per workgroup (filled by a call given timing=(None, None, shape))."""

    def __init__(self):
        self.buf = (ctypes.c_int64 * 3)(0, 0, 0)

    @property
    def launches(self) -> int:
        return int(self.buf[0])

    @property
    def blocks(self) -> int:
        return int(self.buf[1])

    @property
    def threads(self) -> int:
        return int(self.buf[2])


def call_timed(name: str, args: tuple, start: "Event | None", stop: "Event | None",
               shape: "LaunchShape | None" = None) -> int:
    """Run libdcpmerge's `name` with the marshalled `args` through its timed
    twin dcpb_*; returns the status of include/dcpmerge.h (raises
    CaptureError for DCPB_ERR_CAPTURE).  `shape` receives what was launched."""
    fn = getattr(bench_lib(), "dcpb_" + name[len("dcp_"):])
    st = fn(None if start is None else start.handle, None if stop is None else stop.handle, *args,
            None if shape is None else ctypes.cast(shape.buf, ctypes.c_void_p))
    if st == DCPB_ERR_CAPTURE:
        raise CaptureError(name)
    return st


def empty_kernel(blocks: int, threads: int, stream) -> None:
    """Launch a kernel that does nothing, of `blocks` workgroups of `threads`
    threads, on `stream` (a hipStream_t as an int, e.g. torch's cuda_stream)."""
    st = bench_lib().dcpb_empty_kernel(int(blocks), int(threads), stream)
    if st != 0:
        raise RuntimeError("dcpb_empty_kernel failed with status %d" % st)


_hip = None


def hip_runtime():
    """The libamdhip64 mapped into this process (loaded by libdcpmerge's
    dependencies if nothing loaded it before)."""
    global _hip
    if _hip is None:
        bench_lib()
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
