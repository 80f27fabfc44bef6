"""Shared helpers of the GPU tests: host<->device moves of payload arrays and
the acceptance checks against the oracle.

Tolerances (the bar stated for this path):
  combine / in-place outputs:  |got - ref| <= tau_T * M + floor_T, with
      M = sum_i w_i |nan_to_num(o_i)| (fp64, from the oracle) and tau_T =
      1e-5 (fp32), 2^-7 (bf16), 2^-10 (fp16), 2^-4 + 2^-18 (OCP FP8 E4M3:
      half an fp8 ulp, 2^-4 of |out| <= M, plus the fp32 accumulation of up to
      ~60 terms); floor_T is half the spacing of T's subnormals (output
      rounding of tiny values).  M == 0 requires got == 0.
  scaled partials (in-place):  |got - ref| <= tau_T * |ref| + floor_T.
  global LSE:  same class (NaN / +inf / -inf) when the reference is not
      finite; otherwise |got - ref| <= 1e-5 absolute.  Where |ref| >= 128
      half an fp32 ulp of ref is added: G is stored in fp32, and from
      |G| = 128 on half an ulp (2^-17 and up) is no longer small next to
      1e-5.  Below 128 the bar is 1e-5 exactly.

The element-wise checks run as torch CPU ops in fp64 (multi-threaded), so
that whole full-size outputs can be compared row by row.
"""
from __future__ import annotations

import math

import numpy as np
import torch

TAU = {"f32": 1e-5, "bf16": 2.0 ** -7, "f16": 2.0 ** -10, "fp8": 2.0 ** -4 + 2.0 ** -18}
FLOOR = {"f32": 2.0 ** -150, "bf16": 2.0 ** -134, "f16": 2.0 ** -25, "fp8": 2.0 ** -10}
TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}
NP_DT = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16, "fp8": np.uint8}


def to_dev(a: np.ndarray, dt: str, dev) -> torch.Tensor:
    """Storage array (bf16 as uint16 bits, fp8 as uint8 codes) -> device
    tensor of the payload type."""
    if dt == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    if dt == "fp8":
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev).view(torch.float8_e4m3fn)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def to_host(t: torch.Tensor, dt: str) -> np.ndarray:
    """Device tensor -> storage array (bf16 as uint16 bits, fp8 as uint8 codes)."""
    t = t.detach().cpu()
    if dt == "bf16":
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)
    if dt == "fp8":
        return t.contiguous().view(torch.uint8).numpy()
    return t.contiguous().numpy()


def bytes_of(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.uint8).cpu().numpy() if t.dtype != torch.uint8 else t.cpu().numpy()


def decode(a: np.ndarray, dt: str) -> np.ndarray:
    if dt == "bf16":
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if dt == "fp8":
        return torch.from_numpy(np.ascontiguousarray(a)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return a.astype(np.float64)


def _f64(x) -> torch.Tensor:
    if isinstance(x, torch.Tensor):
        return x.detach().cpu().to(torch.float64)
    return torch.from_numpy(np.ascontiguousarray(np.asarray(x, np.float64)))


def _same_shape(g: torch.Tensor, r: torch.Tensor) -> torch.Tensor:
    assert g.numel() == r.numel(), (tuple(g.shape), tuple(r.shape))
    return g.reshape(r.shape)


def _first_bad(bad: torch.Tensor, *arrays, k: int = 5):
    idx = torch.nonzero(bad)[:k]
    vals = [[a[tuple(i.tolist())].item() for i in idx] for a in arrays]
    return idx.tolist(), vals


def check_out(got, ref, mag, dt: str, what: str = "out") -> None:
    """|got - ref| <= tau_T * mag + floor_T element-wise; mag == 0 needs got == 0."""
    g, r, m = _f64(got), _f64(ref), _f64(mag)
    g, m = _same_shape(g, r), _same_shape(m, r)
    bad = ~((g - r).abs() <= TAU[dt] * m + FLOOR[dt])
    bad |= (m == 0) & (g != 0)
    if bool(bad.any()):
        idx, (gv, rv, mv) = _first_bad(bad, g, r, m)
        raise AssertionError("%s: %d of %d elements out of tolerance (tau=%g); first %s: got %s ref %s mag %s" % (
            what, int(bad.sum()), bad.numel(), TAU[dt], idx, gv, rv, mv))


def check_scaled(got, ref, dt: str, what: str = "scaled partial") -> None:
    """|got - ref| <= tau_T * |ref| + floor_T element-wise."""
    g, r = _f64(got), _f64(ref)
    g = _same_shape(g, r)
    bad = ~((g - r).abs() <= TAU[dt] * r.abs() + FLOOR[dt])
    if bool(bad.any()):
        idx, (gv, rv) = _first_bad(bad, g, r)
        raise AssertionError("%s: %d bad; first %s got %s ref %s" % (what, int(bad.sum()), idx, gv, rv))


def ulp32(x: np.ndarray) -> np.ndarray:
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(ax)) - 23)


# |G| from which half an fp32 ulp of G is added to the 1e-5 bound
G_ULP_FROM = 128.0


def lse_tol(ref: np.ndarray) -> np.ndarray:
    """Bound on |got - ref| for a finite global LSE: 1e-5, plus half an fp32
    ulp of ref where |ref| >= 128 (G itself is stored in fp32)."""
    ref = np.asarray(ref, np.float64)
    return 1e-5 + np.where(np.abs(ref) >= G_ULP_FROM, 0.5 * ulp32(ref), 0.0)


def check_lse(got: np.ndarray, ref: np.ndarray) -> None:
    ref = np.asarray(ref, np.float64)
    got = np.asarray(got, np.float64)
    assert got.size == ref.size, (got.shape, ref.shape)
    got = got.reshape(ref.shape)
    nan_r, nan_g = np.isnan(ref), np.isnan(got)
    assert np.array_equal(nan_r, nan_g), "NaN class of G differs at %s" % np.argwhere(nan_r != nan_g)[:5].tolist()
    inf_r = np.isinf(ref)
    assert np.array_equal(got[inf_r], ref[inf_r]), "infinite G differs"
    assert not np.isinf(got[~inf_r & ~nan_r]).any(), "G infinite where the reference is finite"
    fin = np.isfinite(ref)
    err = np.abs(got[fin] - ref[fin])
    tol = lse_tol(ref[fin])
    if not np.all(err <= tol):
        i = int(np.argmax(err - tol))
        raise AssertionError("G off by %g (tol %g) at value %r" % (err[i], tol[i], ref[fin][i]))


def say(*a) -> None:
    print(*a, flush=True)


def finite_frac(x) -> float:
    return float(np.isfinite(x).mean()) if np.size(x) else math.nan
