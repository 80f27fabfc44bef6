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


# The raw HIP stream of a device's current stream, without building a
# torch.cuda.Stream object per call (a public-API fallback where the direct
# query is absent).
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(device: int):
    if _raw_stream is not None:
        return _raw_stream(device)
    return torch.cuda.current_stream(device).cuda_stream


def _invoke(name: str, args: tuple, timing, device: int) -> None:
    """Call `name` of libdcpmerge.so with the marshalled arguments, or its
    timed twin of the measurement library when timing events are given, with
    the tensors' device current (the library launches on the current
    device, on that device's stream)."""
    if device == torch.cuda.current_device():
        ctx = None
    else:
        ctx = torch.cuda.device(device)
        ctx.__enter__()
    try:
        if timing is None:
            st = getattr(_lib.lib(), name)(*args)
        else:
            from . import timing as _timing

            st = _timing.call_timed(name, args, *timing)
    finally:
        if ctx is not None:
            ctx.__exit__(None, None, None)
    _lib.check(st, name)


def _require(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _on_gpu(*ts: Optional[torch.Tensor]) -> int:
    """The device index all given tensors share (ValueError unless they are
    device tensors of one device)."""
    dev = None
    for t in ts:
        if t is None:
            continue
        i = t.get_device()
        if i < 0:
            raise ValueError("libdcpmerge works on device tensors only (got %s)" % t.device)
        if dev is None:
            dev = i
        elif i != dev:
            raise ValueError("all tensors must be on one device")
    return dev


def _payload_ok(t: torch.Tensor, name: str) -> None:
    if t.dtype not in _DTYPE:
        raise ValueError("%s: unsupported dtype %s" % (name, t.dtype))
    # (an empty tensor's strides are arbitrary; the call is then a no-op)
    if not (t.stride(-1) == 1 or t.shape[-1] == 1 or t.numel() == 0):
        raise ValueError("%s: the last (D) dimension must be contiguous" % name)


def _lse_ok(t: torch.Tensor, name: str) -> None:
    if t.dtype != torch.float32:
        raise ValueError("%s: LSE tensors are float32" % name)


def _lead(t: torch.Tensor, nd: int):
    """Shape and strides of t with a leading R dimension: t's own when it has
    nd dimensions, else R = 1 with stride 0 (no view is made)."""
    if t.dim() == nd:
        return tuple(t.shape), t.stride()
    return (1,) + tuple(t.shape), (0,) + t.stride()


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
    dev = _on_gpu(out, lse, dst_o, dst_lse, kv_len)
    nd = 4 if out.dim() == 4 else 3
    if not (out.dim() == nd and lse.dim() == nd - 1 and dst_o.dim() == nd + 1 and dst_lse.dim() == nd):
        raise ValueError("expected out [B,H,D], lse [B,H], dst_o [N,B,Hpr,D], dst_lse [N,B,Hpr] "
                         "(optionally with a leading R)")
    (R, B, H, D), so = _lead(out, 4)
    N = dst_o.shape[-4]
    if not (N >= 1 and H % N == 0):
        raise ValueError("num_heads (%d) must be divisible by the DCP size (%d)" % (H, N))
    Hpr = H // N
    lsh, sl = _lead(lse, 3)
    dsh, do = _lead(dst_o, 5)
    dlsh, dl = _lead(dst_lse, 4)
    if lsh != (R, B, H):
        raise ValueError("lse shape %s != %s" % (tuple(lse.shape), (R, B, H)))
    if dsh != (R, N, B, Hpr, D):
        raise ValueError("dst_o shape %s != %s" % (tuple(dst_o.shape), (R, N, B, Hpr, D)))
    if dlsh != (R, N, B, Hpr):
        raise ValueError("dst_lse shape %s" % (tuple(dst_lse.shape),))
    if dst_o.dtype != out.dtype:
        raise ValueError("dst_o dtype must equal out dtype")
    _payload_ok(out, "out")
    _payload_ok(dst_o, "dst_o")
    _lse_ok(lse, "lse")
    _lse_ok(dst_lse, "dst_lse")
    kl = (0, 0)
    if kv_len is not None:
        ksh, kl = _lead(kv_len, 2)
        if not (kv_len.dtype == torch.int32 and ksh == (R, B) and kv_len.dim() == nd - 2):
            raise ValueError("kv_len must be int32 [R,B] / [B]")
    _invoke("dcp_pack", (
        out.data_ptr(), so[0], so[1], so[2],
        lse.data_ptr(), sl[0], sl[1], sl[2],
        dst_o.data_ptr(), do[0], do[1], do[2], do[3],
        dst_lse.data_ptr(), dl[0], dl[1], dl[2], dl[3],
        kv_len.data_ptr() if kv_len is not None else None, kl[0], kl[1],
        R, N, B, H, D, _dt(out), _stream(dev)), timing, dev)


def dcp_lse_combine(recv_o: torch.Tensor, recv_lse: torch.Tensor, is_lse_base_on_e: bool = True,
                    return_lse: bool = True, out: Optional[torch.Tensor] = None,
                    out_lse: Optional[torch.Tensor] = None, timing=None):
    """LSE-weighted merge over axis 0 of recv_o [N,B,Hpr,D] (any strides) and
    recv_lse [N,B,Hpr].  Returns (out [B,Hpr,D], global LSE [B,Hpr] or None).
    The global LSE is in the input's base.  With a leading R dimension
    (recv_o [R,N,B,Hpr,D]) R merges run at once."""
    dev = _on_gpu(recv_o, recv_lse, out, out_lse)
    batched = recv_o.dim() == 5
    nd = 5 if batched else 4
    if not (recv_o.dim() == nd and recv_lse.dim() == nd - 1):
        raise ValueError("expected recv_o [N,B,Hpr,D] and recv_lse [N,B,Hpr] (optionally with a leading R)")
    (R, N, B, Hpr, D), ro = _lead(recv_o, 5)
    rlsh, rl = _lead(recv_lse, 4)
    if rlsh != (R, N, B, Hpr):
        raise ValueError("recv_lse shape %s" % (tuple(recv_lse.shape),))
    _payload_ok(recv_o, "recv_o")
    _lse_ok(recv_lse, "recv_lse")
    if out is None:
        out = torch.empty((R, B, Hpr, D) if batched else (B, Hpr, D), dtype=recv_o.dtype, device=recv_o.device)
    osh, oo = _lead(out, 4)
    if not (out.dim() == nd - 1 and osh == (R, B, Hpr, D) and out.dtype == recv_o.dtype):
        raise ValueError("bad out tensor")
    _payload_ok(out, "out")
    if return_lse and out_lse is None:
        out_lse = torch.empty((R, B, Hpr) if batched else (B, Hpr), dtype=torch.float32, device=recv_o.device)
    ol = (0, 0, 0)
    if out_lse is not None:
        olsh, ol = _lead(out_lse, 3)
        if not (out_lse.dim() == nd - 2 and olsh == (R, B, Hpr)):
            raise ValueError("bad out_lse shape")
        _lse_ok(out_lse, "out_lse")
    _invoke("dcp_unpack_combine", (
        recv_o.data_ptr(), ro[0], ro[1], ro[2], ro[3],
        recv_lse.data_ptr(), rl[0], rl[1], rl[2], rl[3],
        out.data_ptr(), oo[0], oo[1], oo[2],
        out_lse.data_ptr() if out_lse is not None else None, ol[0], ol[1], ol[2],
        R, N, B, Hpr, D, _dt(recv_o),
        _lib.DCP_LSE_BASE_E if is_lse_base_on_e else _lib.DCP_LSE_BASE_2, _stream(dev)), timing, dev)
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
    dev = _on_gpu(partial, lse, out, out_lse)
    if not (partial.dim() == 4 and lse.dim() == 3):
        raise ValueError("expected partial [P,T,H,D] and lse [N,T,H]")
    P, T, H, D = partial.shape
    N = lse.shape[0]
    h1 = H if h1 is None else h1
    if lse.shape != (N, T, H):
        raise ValueError("lse shape %s" % (tuple(lse.shape),))
    _payload_ok(partial, "partial")
    _lse_ok(lse, "lse")
    if want_out and out is None:
        out = torch.empty((T, max(h1 - h0, 0), D), dtype=partial.dtype, device=partial.device)
    if out is not None:
        if not (out.shape == (T, h1 - h0, D) and out.dtype == partial.dtype):
            raise ValueError("bad out tensor")
        _payload_ok(out, "out")
    if return_lse and out_lse is None:
        out_lse = torch.empty((T, max(h1 - h0, 0)), dtype=torch.float32, device=partial.device)
    if out_lse is not None:
        if out_lse.shape != (T, h1 - h0):
            raise ValueError("bad out_lse shape")
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
        _lib.DCP_LSE_BASE_E if is_lse_base_on_e else _lib.DCP_LSE_BASE_2, _stream(dev)), timing, dev)
    return (out, out_lse) if return_lse else out
