"""ctypes loader of libdcpmerge.so (the C ABI of include/dcpmerge.h).

There is no fallback: if the library is missing or cannot be loaded, every
call raises.  Build it with ``python -m lse_weighted_merge_dcp_amd.csrc.build``.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdcpmerge.so")

DCP_F32, DCP_F16, DCP_BF16, DCP_FP8_E4M3 = 0, 1, 2, 3
DCP_LSE_BASE_E, DCP_LSE_BASE_2 = 0, 1

STATUS = {
    0: "DCP_OK",
    -1: "DCP_ERR_NULL",
    -2: "DCP_ERR_SHAPE",
    -3: "DCP_ERR_HEADS_NOT_DIVISIBLE",
    -4: "DCP_ERR_DTYPE",
    -5: "DCP_ERR_LSE_BASE",
    -6: "DCP_ERR_STRIDE",
    -7: "DCP_ERR_ALIGN",
    -8: "DCP_ERR_HEAD_RANGE",
    -9: "DCP_ERR_LAUNCH",
}

_I64 = ctypes.c_int64
_VP = ctypes.c_void_p
_INT = ctypes.c_int

SIGNATURES = {
    "dcp_lse_pack_dim": ([_INT], _INT),
    "dcp_status_str": ([_INT], ctypes.c_char_p),
    "dcp_pack": ([_VP, _I64, _I64, _I64,
                  _VP, _I64, _I64, _I64,
                  _VP, _I64, _I64, _I64, _I64,
                  _VP, _I64, _I64, _I64, _I64,
                  _VP, _I64, _I64,
                  _I64, _I64, _I64, _I64, _I64,
                  _INT, _VP], _INT),
    "dcp_unpack_combine": ([_VP, _I64, _I64, _I64, _I64,
                            _VP, _I64, _I64, _I64, _I64,
                            _VP, _I64, _I64, _I64,
                            _VP, _I64, _I64, _I64,
                            _I64, _I64, _I64, _I64, _I64,
                            _INT, _INT, _VP], _INT),
    "dcp_lse_combine_inplace": ([_VP, _I64, _I64, _I64,
                                 _VP, _I64, _I64, _I64,
                                 _I64, _I64,
                                 _VP, _I64, _I64,
                                 _VP, _I64, _I64,
                                 _I64, _I64, _I64,
                                 _I64, _I64, _I64,
                                 _INT, _INT, _VP], _INT),
}

_lib = None


class DcpError(ValueError):
    """A libdcpmerge call rejected its arguments (nothing was enqueued)."""

    def __init__(self, status: int, fn: str):
        self.status = status
        super().__init__("%s failed: %s" % (fn, STATUS.get(status, status)))


class DcpLaunchError(RuntimeError):
    """The HIP kernel launch failed."""


def lib():
    """The loaded library (loads it on first use; raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                "libdcpmerge.so is not built (expected at %s); run "
                "`python -m lse_weighted_merge_dcp_amd.csrc.build`" % LIB_PATH)
        h = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in SIGNATURES.items():
            fn = getattr(h, name)
            fn.argtypes = args
            fn.restype = res
        _lib = h
    return _lib


def check(status: int, fn: str) -> None:
    if status == -9:
        raise DcpLaunchError("%s failed: DCP_ERR_LAUNCH" % fn)
    if status != 0:
        raise DcpError(status, fn)
