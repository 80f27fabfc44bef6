"""Python API of libdcpmerge, shaped like the pages' calls.

Argument marshalling only: tensors become device pointers, element strides,
sizes and the current HIP stream; every step runs in the HIP kernels of
libdcpmerge.so.  PyTorch provides device memory (outputs are allocated with
torch.empty) and streams.  There is no CPU or PyTorch fallback.

  dcp_pack_a2a_send(out, lse, dst_o, dst_lse)
      sglang PR #34651 report, 实现拆解 item 1 (stride-driven pack)
  dcp_lse_combine(recv_o, recv_lse, is_lse_base_on_e, return_lse)
      sglang PR #34651 report, 实现拆解 item 3; vLLM PR #41160 report, 实现拆解 items 1-3
  cp_lse_combine_inplace(partial, lse, h0, h1, ...)
      sglang PR #34213 report, code excerpt of cp_lse_ag_out_rs_mha
  lse_pack_dim(dtype), interleaved_views(send, D)
      vLLM PR #41160 report, 实现拆解 item 2; sglang PR #34651 report, 实现拆解 item 2

Every entry point also accepts a leading R dimension (R independent calls
in one launch, e.g. all simulated ranks stacked in one GPU's memory).

The three compute calls take an optional `timing=(start, stop)` pair of
timing.Event for measurement: that one call then runs the same kernels
through the separate measurement library (timing.py), with the events on
the kernels' own dispatches.  Without it (the default) the call goes to
libdcpmerge.so, which keeps no state.
"""
from __future__ import annotations

from typing import Optional, Tuple

import torch

from . import _lib

_DTYPE = {torch.float32: _lib.DCP_F32, torch.float16: _lib.DCP_F16, torch.bfloat16: _lib.DCP_BF16,
          torch.float8_e4m3fn: _lib.DCP_FP8_E4M3}


def _dt(t: torch.Tensor) -> int:
    return _DTYPE.get(t.dtype, -1)


def _stream(t: torch.Tensor):
    return torch.cuda.current_stream(t.device).cuda_stream


def _invoke(name: str, args: tuple, timing, device: torch.device) -> None:
    """Call `name` of libdcpmerge.so with the marshalled arguments, or its
    timed twin of the measurement library when timing events are given, with
    the tensors' device current (the library launches on the current
    device, on that device's stream)."""
    with torch.cuda.device(device):
        if timing is None:
            st = getattr(_lib.lib(), name)(*args)
        else:
            from . import timing as _timing

            st = _timing.call_timed(name, args, *timing)
    _lib.check(st, name)


def _require(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _on_gpu(*ts: Optional[torch.Tensor]) -> None:
    dev = None
    for t in ts:
        if t is None:
            continue
        _require(t.is_cuda, "libdcpmerge works on device tensors only (got %s)" % t.device)
        _require(dev is None or t.device == dev, "all tensors must be on one device")
        dev = t.device


def _payload_ok(t: torch.Tensor, name: str) -> None:
    _require(t.dtype in _DTYPE, "%s: unsupported dtype %s" % (name, t.dtype))
    # (an empty tensor's strides are arbitrary; the call is then a no-op)
    _require(t.numel() == 0 or t.shape[-1] == 1 or t.stride(-1) == 1,
             "%s: the last (D) dimension must be contiguous" % name)


def _lse_ok(t: torch.Tensor, name: str) -> None:
    _require(t.dtype == torch.float32, "%s: LSE tensors are float32" % name)


def lse_pack_dim(dtype: torch.dtype) -> int:
    """Payload elements one fp32 LSE occupies at the tail of a row: 1 for
    float32, 2 for float16/bfloat16, 4 for float8_e4m3fn.  Other dtypes raise
    ValueError."""
    code = _lib.lib().dcp_lse_pack_dim(_DTYPE.get(dtype, -1))
    if code < 0:
        raise ValueError("no LSE pack dim for dtype %s" % dtype)
    return code


def interleaved_views(send: torch.Tensor, D: int) -> Tuple[torch.Tensor, torch.Tensor]:
    """Payload view send[..., :D] and the fp32 LSE-word view of an
    interleaved send buffer send[..., D + lpd] (one all-to-all moves both):
    the LSE is fp32 word D / lpd of each row's fp32 reinterpretation."""
    lpd = lse_pack_dim(send.dtype)
    _require(D % lpd == 0, "D (%d) must be a multiple of the LSE pack dim (%d)" % (D, lpd))
    _require(send.shape[-1] == D + lpd, "send rows must hold D + lpd = %d elements" % (D + lpd))
    _require(send.is_contiguous(), "send buffer must be contiguous")
    if send.numel() == 0:
        # nothing to address; an empty tensor's strides may not allow the view
        send = torch.empty(send.shape, dtype=send.dtype, device=send.device)
    words = send.view(torch.float32)
    return send[..., :D], words[..., D // lpd]


def dcp_pack_a2a_send(out: torch.Tensor, lse: torch.Tensor, dst_o: torch.Tensor, dst_lse: torch.Tensor,
                      kv_len: Optional[torch.Tensor] = None, timing=None) -> None:
    """Scatter out [B,H,D] / lse [B,H] into dst_o [N,B,H/N,D] / dst_lse
    [N,B,H/N] (any strides): head h goes to peer h // (H/N) as local head
    h % (H/N).  With a leading R dimension on all four, R packs run at once.
    kv_len ([B] or [R,B] int32, optional): tokens whose rank-local KV length
    is 0 are sent as the neutral pair (0, -inf) instead of the partial (the
    fixup_zero_kv_rows step of sglang PR #33926 report, 实现拆解 item 3)."""
    _on_gpu(out, lse, dst_o, dst_lse, kv_len)
    batched = out.dim() == 4
    if not batched:
        out, lse, dst_o, dst_lse = out[None], lse[None], dst_o[None], dst_lse[None]
        kv_len = kv_len[None] if kv_len is not None else None
    _require(out.dim() == 4 and lse.dim() == 3 and dst_o.dim() == 5 and dst_lse.dim() == 4,
             "expected out [B,H,D], lse [B,H], dst_o [N,B,Hpr,D], dst_lse [N,B,Hpr] (optionally with a leading R)")
    R, B, H, D = out.shape
    N = dst_o.shape[1]
    _require(N >= 1 and H % N == 0, "num_heads (%d) must be divisible by the DCP size (%d)" % (H, N))
    Hpr = H // N
    _require(tuple(lse.shape) == (R, B, H), "lse shape %s != %s" % (tuple(lse.shape), (R, B, H)))
    _require(tuple(dst_o.shape) == (R, N, B, Hpr, D), "dst_o shape %s != %s" % (tuple(dst_o.shape), (R, N, B, Hpr, D)))
    _require(tuple(dst_lse.shape) == (R, N, B, Hpr), "dst_lse shape %s" % (tuple(dst_lse.shape),))
    _require(dst_o.dtype == out.dtype, "dst_o dtype must equal out dtype")
    _payload_ok(out, "out")
    _payload_ok(dst_o, "dst_o")
    _lse_ok(lse, "lse")
    _lse_ok(dst_lse, "dst_lse")
    kl = (0, 0)
    if kv_len is not None:
        _require(kv_len.dtype == torch.int32 and tuple(kv_len.shape) == (R, B), "kv_len must be int32 [R,B] / [B]")
        kl = kv_len.stride()
    so, sl, do, dl = out.stride(), lse.stride(), dst_o.stride(), dst_lse.stride()
    _invoke("dcp_pack", (
        out.data_ptr(), so[0], so[1], so[2],
        lse.data_ptr(), sl[0], sl[1], sl[2],
        dst_o.data_ptr(), do[0], do[1], do[2], do[3],
        dst_lse.data_ptr(), dl[0], dl[1], dl[2], dl[3],
        kv_len.data_ptr() if kv_len is not None else None, kl[0], kl[1],
        R, N, B, H, D, _dt(out), _stream(out)), timing, out.device)


def dcp_lse_combine(recv_o: torch.Tensor, recv_lse: torch.Tensor, is_lse_base_on_e: bool = True,
                    return_lse: bool = True, out: Optional[torch.Tensor] = None,
                    out_lse: Optional[torch.Tensor] = None, timing=None):
    """LSE-weighted merge over axis 0 of recv_o [N,B,Hpr,D] (any strides) and
    recv_lse [N,B,Hpr].  Returns (out [B,Hpr,D], global LSE [B,Hpr] or None).
    The global LSE is in the input's base.  With a leading R dimension
    (recv_o [R,N,B,Hpr,D]) R merges run at once."""
    _on_gpu(recv_o, recv_lse, out, out_lse)
    batched = recv_o.dim() == 5
    if not batched:
        recv_o, recv_lse = recv_o[None], recv_lse[None]
        out = out[None] if out is not None else None
        out_lse = out_lse[None] if out_lse is not None else None
    _require(recv_o.dim() == 5 and recv_lse.dim() == 4,
             "expected recv_o [N,B,Hpr,D] and recv_lse [N,B,Hpr] (optionally with a leading R)")
    R, N, B, Hpr, D = recv_o.shape
    _require(tuple(recv_lse.shape) == (R, N, B, Hpr), "recv_lse shape %s" % (tuple(recv_lse.shape),))
    _payload_ok(recv_o, "recv_o")
    _lse_ok(recv_lse, "recv_lse")
    if out is None:
        out = torch.empty((R, B, Hpr, D), dtype=recv_o.dtype, device=recv_o.device)
    _require(tuple(out.shape) == (R, B, Hpr, D) and out.dtype == recv_o.dtype, "bad out tensor")
    _payload_ok(out, "out")
    if return_lse and out_lse is None:
        out_lse = torch.empty((R, B, Hpr), dtype=torch.float32, device=recv_o.device)
    if out_lse is not None:
        _require(tuple(out_lse.shape) == (R, B, Hpr), "bad out_lse shape")
        _lse_ok(out_lse, "out_lse")
    ro, rl, oo = recv_o.stride(), recv_lse.stride(), out.stride()
    ol = out_lse.stride() if out_lse is not None else (0, 0, 0)
    _invoke("dcp_unpack_combine", (
        recv_o.data_ptr(), ro[0], ro[1], ro[2], ro[3],
        recv_lse.data_ptr(), rl[0], rl[1], rl[2], rl[3],
        out.data_ptr(), oo[0], oo[1], oo[2],
        out_lse.data_ptr() if out_lse is not None else None, ol[0], ol[1], ol[2],
        R, N, B, Hpr, D, _dt(recv_o),
        _lib.DCP_LSE_BASE_E if is_lse_base_on_e else _lib.DCP_LSE_BASE_2, _stream(recv_o)), timing, recv_o.device)
    if not batched:
        out = out[0]
        out_lse = out_lse[0] if out_lse is not None else None
    return out, (out_lse if return_lse else None)


def cp_lse_combine_inplace(partial: torch.Tensor, lse: torch.Tensor, h0: int = 0, h1: Optional[int] = None,
                           rank0: int = 0, is_lse_base_on_e: bool = True, return_lse: bool = False,
                           out: Optional[torch.Tensor] = None, out_lse: Optional[torch.Tensor] = None,
                           want_out: bool = True, timing=None):
    """In-place merge: partial [P,T,H,D] holds ranks rank0..rank0+P-1 of the
    N = lse.shape[0] ranks; lse [N,T,H].  Every held partial is overwritten
    with nan_to_num(o) * w, and out [T,h1-h0,D] = sum of the held scaled
    partials over heads [h0, h1).  Returns out, or (out, global LSE slice)
    if return_lse.  want_out=False only scales (out is None)."""
    _on_gpu(partial, lse, out, out_lse)
    _require(partial.dim() == 4 and lse.dim() == 3, "expected partial [P,T,H,D] and lse [N,T,H]")
    P, T, H, D = partial.shape
    N = lse.shape[0]
    h1 = H if h1 is None else h1
    _require(tuple(lse.shape) == (N, T, H), "lse shape %s" % (tuple(lse.shape),))
    _payload_ok(partial, "partial")
    _lse_ok(lse, "lse")
    if want_out and out is None:
        out = torch.empty((T, max(h1 - h0, 0), D), dtype=partial.dtype, device=partial.device)
    if out is not None:
        _require(tuple(out.shape) == (T, h1 - h0, D) and out.dtype == partial.dtype, "bad out tensor")
        _payload_ok(out, "out")
    if return_lse and out_lse is None:
        out_lse = torch.empty((T, max(h1 - h0, 0)), dtype=torch.float32, device=partial.device)
    if out_lse is not None:
        _require(tuple(out_lse.shape) == (T, h1 - h0), "bad out_lse shape")
        _lse_ok(out_lse, "out_lse")
    ps, ls = partial.stride(), lse.stride()
    os_ = out.stride() if out is not None else (0, 0, 0)
    ols = out_lse.stride() if out_lse is not None else (0, 0)
    _invoke("dcp_lse_combine_inplace", (
        partial.data_ptr(), ps[0], ps[1], ps[2],
        lse.data_ptr(), ls[0], ls[1], ls[2],
        h0, h1,
        out.data_ptr() if out is not None else None, os_[0], os_[1],
        out_lse.data_ptr() if out_lse is not None else None, ols[0], ols[1],
        N, P, rank0, T, H, D, _dt(partial),
        _lib.DCP_LSE_BASE_E if is_lse_base_on_e else _lib.DCP_LSE_BASE_2, _stream(partial)), timing, partial.device)
    return (out, out_lse) if return_lse else out
