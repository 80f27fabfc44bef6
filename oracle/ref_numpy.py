"""A second CPU oracle, in plain NumPy -- TEST INFRASTRUCTURE ONLY.

Only ``tests/`` may import this module.  It is written independently of
``dcp_oracle.c`` (it shares no code with it, nor with the HIP library) so
that the two fp64 oracles can check each other: the merge is an exact
LSE-weighted reduction (vLLM PR #41160 report, 功能与动机), so two correct
fp64 implementations agree to rounding (about 1e-15 relative).

Where dcp_oracle.c shifts by the maximum and sums powers, this twin folds
the ranks with NumPy's pairwise log-add-exp (``np.logaddexp.reduce`` in base
e, ``np.logaddexp2.reduce`` in base 2), which gives logsumexp's special
values by itself: any NaN gives NaN, else any +inf gives +inf, and all -inf
give -inf (the semantics of the torch.logsumexp call in the code excerpt of
cp_lse_ag_out_rs_mha, sglang PR #34213 report).  The weights and guards
follow that same excerpt: w_i = nan_to_num(base^(l_i - G)), o'_i =
nan_to_num(o_i), out = sum_i w_i o'_i; a single rank is returned unchanged
(its world_size == 1 shortcut).  The base flag is the one of sglang PR #33926
report, 实现拆解 item 4.

Payload decoding to fp64 is exact and done with library conversions: numpy
for fp32/fp16, a 16-bit shift for bf16, torch's float8_e4m3fn for fp8.
"""
from __future__ import annotations

import numpy as np
import torch


def decode(a: np.ndarray, dt: str) -> np.ndarray:
    """Exact fp64 values of a payload array (bf16 as raw uint16 bits, fp8
    as raw uint8 codes)."""
    if dt in ("f32", "f16"):
        return np.asarray(a).astype(np.float64)
    if dt == "bf16":
        return (np.asarray(a, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dt == "fp8":
        codes = torch.from_numpy(np.ascontiguousarray(a, np.uint8))
        return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    raise ValueError(dt)


def global_lse(lse: np.ndarray, base2: bool) -> np.ndarray:
    """log_base sum_i base^lse[i] over axis 0, folded pairwise."""
    l = np.asarray(lse, np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        return (np.logaddexp2 if base2 else np.logaddexp).reduce(l, axis=0)


def weights(lse: np.ndarray, G: np.ndarray, base2: bool) -> np.ndarray:
    """w_i = nan_to_num(base^(lse_i - G)), NaN and +-inf -> 0."""
    l = np.asarray(lse, np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        x = l - G[None]
        w = np.exp2(x) if base2 else np.exp(x)
    return np.nan_to_num(w, nan=0.0, posinf=0.0, neginf=0.0)


def combine(recv_o: np.ndarray, recv_lse: np.ndarray, dt: str, base2: bool):
    """Out-of-place merge over axis 0 of recv_o [N, ...rows, D] and
    recv_lse [N, ...rows].  Returns (out [...rows, D], G [...rows]) in fp64."""
    o = decode(recv_o, dt)
    l = np.asarray(recv_lse, np.float64)
    if o.shape[0] == 1:
        return o[0], l[0]
    G = global_lse(l, base2)
    w = weights(l, G, base2)
    o = np.nan_to_num(o, nan=0.0, posinf=0.0, neginf=0.0)
    return np.einsum("n...,n...d->...d", w, o), G


def inplace(partial: np.ndarray, lse: np.ndarray, dt: str, base2: bool, rank0: int = 0,
            h0: int = 0, h1: int | None = None):
    """The in-place merge: partial [P, T, H, D] holds ranks rank0..rank0+P-1
    of the N = lse.shape[0] ranks.  Returns (scaled [P, T, H, D], out
    [T, h1-h0, D], G [T, h1-h0]) in fp64: scaled_j = nan_to_num(o_j) *
    w_{rank0+j}, out = sum_j scaled_j over heads [h0, h1)."""
    o = decode(partial, dt)
    l = np.asarray(lse, np.float64)
    P, H = o.shape[0], o.shape[2]
    h1 = H if h1 is None else h1
    if l.shape[0] == 1:
        return o.copy(), o[0][:, h0:h1], l[0][:, h0:h1]
    G = global_lse(l, base2)
    w = weights(l, G, base2)[rank0:rank0 + P]
    scaled = np.nan_to_num(o, nan=0.0, posinf=0.0, neginf=0.0) * w[..., None]
    out = scaled.sum(axis=0)
    return scaled, out[:, h0:h1], G[:, h0:h1]
