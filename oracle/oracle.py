"""fp64 CPU oracle for the DCP partial-merge path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  It shares no code with the HIP library
(``lse_weighted_merge_dcp_amd``) and never imports it; the product path never
imports this.

The arithmetic lives in ``dcp_oracle.c`` (plain fp64 loops).  This wrapper
only moves numpy arrays in and out:

* payload arrays are numpy views of any strides; dtype tags are ``"f32"``,
  ``"f16"``, ``"bf16"`` (carried as raw ``uint16`` bits) and ``"fp8"`` (OCP
  FP8 E4M3, carried as raw ``uint8`` codes);
* LSE arrays are ``float32`` views of any strides;
* the combine and in-place functions decode the payload to fp64 exactly
  (every fp32/fp16/bf16/fp8 value is an fp64 value) before calling C.

Citations (page title, then section):
  sglang PR #34651 report -- 实现拆解 items 1-3 and its split-layout test excerpt;
  vLLM PR #41160 report -- 实现拆解 items 1-3;
  sglang PR #33926 report -- 实现拆解 items 3-4;
  sglang PR #34213 report -- code excerpt of cp_lse_ag_out_rs_mha.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dcp_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libdcp_oracle.so")
_lib = None

ESIZE = {"f32": 4, "f16": 2, "bf16": 2, "fp8": 1}


def compile_source(src: str, out: str) -> str:
    """gcc -O2 -fopenmp of an oracle C source into a shared library."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.check_call(
        ["gcc", "-O2", "-fopenmp", "-fno-fast-math", "-shared", "-fPIC",
         "-Wall", "-Wextra", src, "-o", tmp, "-lm"])
    os.replace(tmp, out)
    return out


def build(force: bool = False) -> str:
    """Compile dcp_oracle.c (fp64, OpenMP) next to this file."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        compile_source(_SRC, _LIB_PATH)
    return _LIB_PATH


def load_library(path: str):
    """Load a compiled oracle library (the default one, or a test's variant)."""
    lib = ctypes.CDLL(path)
    i64, vp, c_int = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    lib.orc_pack.argtypes = [vp, i64, i64, i64, vp, i64, i64,
                             vp, i64, i64, i64, i64, vp, i64, i64, i64,
                             vp, i64,
                             i64, i64, i64, i64, i64]
    lib.orc_pack.restype = None
    lib.orc_combine.argtypes = [vp, vp, i64, i64, i64, c_int, vp, vp, vp, vp]
    lib.orc_combine.restype = None
    lib.orc_inplace.argtypes = [vp, vp, i64, i64, i64, i64, i64, c_int, vp, vp, vp, vp]
    lib.orc_inplace.restype = None
    lib.orc_num_threads.argtypes = []
    lib.orc_num_threads.restype = c_int
    lib.orc_set_num_threads.argtypes = [c_int]
    lib.orc_set_num_threads.restype = None
    return lib


def _load(lib=None):
    global _lib
    if lib is not None:
        return lib
    if _lib is None:
        # DCP_ORACLE_LIB names another build of dcp_oracle.c to use instead
        # (the tests run the pins against a sanitizer build this way)
        other = os.environ.get("DCP_ORACLE_LIB")
        if other:
            _lib = load_library(other)
        else:
            build()
            _lib = load_library(_LIB_PATH)
    return _lib


def num_threads() -> int:
    return int(_load().orc_num_threads())


def set_num_threads(n: int) -> None:
    """Threads of the oracle's parallel loops (timing only; results do not
    depend on it: every loop iteration is an independent row)."""
    _load().orc_set_num_threads(int(n))


def _ptr(a: np.ndarray) -> int:
    return a.__array_interface__["data"][0]


# --------------------------------------------------------------------------
# exact decoding of the payload element types to fp64
# --------------------------------------------------------------------------
def fp8_e4m3_values() -> np.ndarray:
    """fp64 value of each of the 256 codes of OCP FP8 E4M3 (e4m3fn), from the
    format's definition: bit 7 the sign, bits 6..3 the exponent e (bias 7),
    bits 2..0 the mantissa m; e = 0 encodes the subnormals (m / 8) * 2^-6,
    e = 15 with m = 7 is NaN, and there are no infinities (so e = 15, m < 7
    are ordinary numbers, the largest 1.75 * 2^8 = 448).  The pages name fp8
    only as a payload type still to be reviewed (sglang PR #34651 report,
    风险与影响; vLLM PR #41160 report, 风险与影响); the format itself is the
    OCP 8-bit floating-point specification's E4M3."""
    t = np.empty(256, np.float64)
    for c in range(256):
        sign = -1.0 if c & 0x80 else 1.0
        e, m = (c >> 3) & 0xF, c & 0x7
        if e == 0xF and m == 0x7:
            t[c] = math.nan
        elif e == 0:
            t[c] = sign * (m / 8.0) * 2.0 ** -6
        else:
            t[c] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return t


def to_f64(a: np.ndarray, dt: str) -> np.ndarray:
    """Exact fp64 value of every element (bf16 given as raw uint16 bits,
    fp8 as raw uint8 codes)."""
    if dt == "f32":
        assert a.dtype == np.float32
        return a.astype(np.float64)
    if dt == "f16":
        assert a.dtype == np.float16
        return a.astype(np.float64)
    if dt == "bf16":
        assert a.dtype == np.uint16
        # a bf16 value is the fp32 value whose upper 16 bits are these bits
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if dt == "fp8":
        assert a.dtype == np.uint8
        return fp8_e4m3_values()[a]
    raise ValueError(dt)


# --------------------------------------------------------------------------
# pack
# --------------------------------------------------------------------------
def pack(src_o: np.ndarray, src_lse: np.ndarray, dst_o: np.ndarray, dst_lse: np.ndarray, N: int,
         lib=None, kv_len: np.ndarray | None = None) -> None:
    """Scatter one rank's [B,H,D] payload and [B,H] fp32 LSE into the per-peer
    views dst_o [N,B,H/N,D] and dst_lse [N,B,H/N] (any strides, written in
    place).  Bit copy.  sglang PR #34651 report, 实现拆解 item 1.  With kv_len
    ([B] int32), a token whose rank-local KV length is 0 is sent as the
    neutral pair (0, -inf) (sglang PR #33926 report, 实现拆解 item 3)."""
    B, H, D = src_o.shape
    assert H % N == 0
    Hpr = H // N
    assert dst_o.shape == (N, B, Hpr, D) and dst_lse.shape == (N, B, Hpr)
    assert src_lse.shape == (B, H) and src_lse.itemsize == 4 and dst_lse.itemsize == 4
    assert src_o.itemsize == dst_o.itemsize
    assert dst_o.flags.writeable and dst_lse.flags.writeable
    kv_ptr, kv_stride = None, 0
    if kv_len is not None:
        assert kv_len.dtype == np.int32 and kv_len.shape == (B,)
        kv_ptr, kv_stride = _ptr(kv_len), kv_len.strides[0]
    _load(lib).orc_pack(_ptr(src_o), *src_o.strides, _ptr(src_lse), *src_lse.strides,
                        _ptr(dst_o), *dst_o.strides, _ptr(dst_lse), *dst_lse.strides,
                        kv_ptr, kv_stride, N, B, H, D, src_o.itemsize)


# --------------------------------------------------------------------------
# combine (out of place)
# --------------------------------------------------------------------------
def combine(recv_o: np.ndarray, recv_lse: np.ndarray, dt: str, base2: bool, lib=None):
    """LSE-weighted merge over axis 0 of recv_o [N,B,Hpr,D] / recv_lse [N,B,Hpr].

    Returns (out [B,Hpr,D] fp64, G [B,Hpr] fp64, mag [B,Hpr,D] fp64, w [N,B,Hpr]).
    ``mag`` = sum_i w_i*|nan_to_num(o_i)|, the size of the terms summed, used
    for the tolerance.  sglang PR #34651 report 实现拆解 item 3; vLLM PR #41160
    report 实现拆解 item 1; guards from sglang PR #34213 report's code excerpt.
    """
    N, B, Hpr, D = recv_o.shape
    assert recv_lse.shape == (N, B, Hpr) and recv_lse.dtype == np.float32
    rows = B * Hpr
    o = np.ascontiguousarray(to_f64(recv_o, dt).reshape(N, rows, D))
    l = np.ascontiguousarray(recv_lse.astype(np.float64).reshape(N, rows))
    out = np.empty((rows, D), np.float64)
    g = np.empty((rows,), np.float64)
    mag = np.empty((rows, D), np.float64)
    w = np.empty((N, rows), np.float64)
    _load(lib).orc_combine(_ptr(o), _ptr(l), N, rows, D, int(bool(base2)), _ptr(out), _ptr(g), _ptr(mag), _ptr(w))
    return out.reshape(B, Hpr, D), g.reshape(B, Hpr), mag.reshape(B, Hpr, D), w.reshape(N, B, Hpr)


# --------------------------------------------------------------------------
# in-place merge
# --------------------------------------------------------------------------
def inplace(partial: np.ndarray, lse: np.ndarray, dt: str, base2: bool, rank0: int = 0,
            h0: int = 0, h1: int | None = None, lib=None):
    """In-place merge of sglang PR #34213 report's cp_lse_ag_out_rs_mha.

    partial [P,T,H,D] (the partials held, partial j = rank rank0 + j),
    lse [N,T,H] fp32 (every rank's LSE).  Returns
      scaled [P,T,H,D] fp64  -- the partial buffer's expected contents after the call,
      out    [T,h1-h0,D]     -- sum over the held partials, heads [h0, h1),
      G      [T,h1-h0]       -- global LSE, same heads,
      mag    [T,h1-h0,D]     -- sum of |scaled| (tolerance scale).
    """
    P, T, H, D = partial.shape
    N = lse.shape[0]
    assert lse.shape == (N, T, H) and lse.dtype == np.float32
    assert 1 <= P and 0 <= rank0 and rank0 + P <= N
    h1 = H if h1 is None else h1
    rows = T * H
    o = np.ascontiguousarray(to_f64(partial, dt).reshape(P, rows, D))
    l = np.ascontiguousarray(lse.astype(np.float64).reshape(N, rows))
    scaled = np.empty((P, rows, D), np.float64)
    out = np.empty((rows, D), np.float64)
    g = np.empty((rows,), np.float64)
    mag = np.empty((rows, D), np.float64)
    _load(lib).orc_inplace(_ptr(o), _ptr(l), N, P, rank0, rows, D, int(bool(base2)),
                        _ptr(scaled), _ptr(out), _ptr(g), _ptr(mag))
    out = out.reshape(T, H, D)[:, h0:h1]
    g = g.reshape(T, H)[:, h0:h1]
    mag = mag.reshape(T, H, D)[:, h0:h1]
    return scaled.reshape(P, T, H, D), out, g, mag


# --------------------------------------------------------------------------
# layout helpers (numpy views of a host send buffer; oracle-side only)
# --------------------------------------------------------------------------
def interleaved_views_np(send: np.ndarray, D: int, dt: str):
    """Payload view [..., :D] and fp32 LSE word view of an interleaved send
    buffer [..., D + 4/e] in the payload's own element type.  The LSE is the
    fp32 word D/lpd of each row's fp32 reinterpretation (sglang PR #34651
    report, 实现拆解 item 2)."""
    e = ESIZE[dt]
    lpd = 4 // e
    assert D % lpd == 0 and send.shape[-1] == D + lpd and send.flags.c_contiguous
    payload = send[..., :D]
    words = send.view(np.float32)
    return payload, words[..., D // lpd]
