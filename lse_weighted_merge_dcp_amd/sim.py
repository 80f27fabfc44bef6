"""Single-GPU simulation of a DCP group: all N ranks stacked in one GPU's memory.

The exchange between pack and combine (an all-to-all across ranks) is not a
step of this library; here it is simulated without a second GPU:

* interleaved (pynccl-style) layout: every source's send buffer
  [N, B, Hpr, D + lpd] lives in one allocation send[src, peer, ...].  After
  the all-to-all, destination p holds chunk p of every source, which is the
  zero-copy view send[:, p]; all destinations together are send.transpose(0, 1).
* split (FlashInfer-style) layout: partial_o [B, Hpr, N, D] and stats
  [B, Hpr, N, 2] per rank, peer axis inside the heads.  The exchange moves
  o_out[dst, b, hl, src] = partial_o[src, b, hl, dst] (stats slot 1 as opaque
  bytes); it is simulated with a device copy that stands in for the
  collective and is never timed as part of the merge.

sglang PR #34651 report, 实现拆解 items 2-3 (both layouts and their views).
"""
from __future__ import annotations

import torch

from . import ops


class StackedInterleaved:
    """Peer-outer interleaved send buffers of N ranks, stacked."""

    def __init__(self, N: int, B: int, H: int, D: int, dtype: torch.dtype, device):
        assert H % N == 0
        self.N, self.B, self.H, self.D = N, B, H, D
        self.lpd = ops.lse_pack_dim(dtype)
        self.send = torch.empty((N, N, B, H // N, D + self.lpd), dtype=dtype, device=device)
        self.payload, self.words = ops.interleaved_views(self.send, D)

    def pack(self, out: torch.Tensor, lse: torch.Tensor, kv_len=None, timing=None) -> None:
        """out [N,B,H,D], lse [N,B,H] (kv_len [N,B] int32 optional): every rank
        packs its own send buffer (one launch)."""
        ops.dcp_pack_a2a_send(out, lse, self.payload, self.words, kv_len=kv_len, timing=timing)

    def pack_rank(self, r: int, out: torch.Tensor, lse: torch.Tensor, kv_len=None, timing=None) -> None:
        """Rank r's own pack at its real shape: out [B,H,D], lse [B,H] (kv_len
        [B] int32 optional)."""
        ops.dcp_pack_a2a_send(out, lse, self.payload[r], self.words[r], kv_len=kv_len, timing=timing)

    def recv(self):
        """Received buffers of all destinations: [dst, src, B, Hpr, D] and [dst, src, B, Hpr]."""
        return self.payload.transpose(0, 1), self.words.transpose(0, 1)

    def combine_dest(self, p: int, is_lse_base_on_e: bool, out=None, out_lse=None, timing=None):
        """Destination p's own combine at its real shape (its received [N, B, Hpr, D])."""
        ro, rl = self.recv()
        return ops.dcp_lse_combine(ro[p], rl[p], is_lse_base_on_e=is_lse_base_on_e, out=out, out_lse=out_lse,
                                   timing=timing)

    def combine(self, is_lse_base_on_e: bool, return_lse: bool = True, out=None, out_lse=None, timing=None):
        ro, rl = self.recv()
        return ops.dcp_lse_combine(ro, rl, is_lse_base_on_e=is_lse_base_on_e, return_lse=return_lse,
                                   out=out, out_lse=out_lse, timing=timing)


class StackedSplit:
    """FlashInfer-shaped split buffers of N ranks, stacked."""

    def __init__(self, N: int, B: int, H: int, D: int, dtype: torch.dtype, device):
        assert H % N == 0
        Hpr = H // N
        self.N, self.B, self.H, self.D = N, B, H, D
        self.partial_o = torch.empty((N, B, Hpr, N, D), dtype=dtype, device=device)
        self.stats = torch.empty((N, B, Hpr, N, 2), dtype=torch.float32, device=device)
        self.o_out = torch.empty_like(self.partial_o)
        self.stats_out = torch.empty_like(self.stats)

    def pack(self, out: torch.Tensor, lse: torch.Tensor, kv_len=None, timing=None) -> None:
        ops.dcp_pack_a2a_send(out, lse, self.partial_o.permute(0, 3, 1, 2, 4),
                              self.stats[..., 0].permute(0, 3, 1, 2), kv_len=kv_len, timing=timing)

    def pack_rank(self, r: int, out: torch.Tensor, lse: torch.Tensor, kv_len=None, timing=None) -> None:
        """Rank r's own pack at its real shape: out [B,H,D], lse [B,H] (kv_len
        [B] int32 optional)."""
        ops.dcp_pack_a2a_send(out, lse, self.partial_o[r].permute(2, 0, 1, 3), self.stats[r][..., 0].permute(2, 0, 1),
                              kv_len=kv_len, timing=timing)

    def exchange(self) -> None:
        """Stand-in for the all-to-all: o_out[dst, b, hl, src] = partial_o[src, b, hl, dst]."""
        self.o_out.copy_(self.partial_o.permute(3, 1, 2, 0, 4))
        self.stats_out.copy_(self.stats.permute(3, 1, 2, 0, 4))

    def recv(self):
        """Strided receive views [dst, src, B, Hpr, D] and [dst, src, B, Hpr] (no copy)."""
        return self.o_out.permute(0, 3, 1, 2, 4), self.stats_out[..., 0].permute(0, 3, 1, 2)

    def combine(self, is_lse_base_on_e: bool, return_lse: bool = True, out=None, out_lse=None, timing=None):
        ro, rl = self.recv()
        return ops.dcp_lse_combine(ro, rl, is_lse_base_on_e=is_lse_base_on_e, return_lse=return_lse,
                                   out=out, out_lse=out_lse, timing=timing)

    def combine_dest(self, p: int, is_lse_base_on_e: bool, out=None, out_lse=None, timing=None):
        """Destination p's own combine at its real shape (its received [N, B, Hpr, D])."""
        ro, rl = self.recv()
        return ops.dcp_lse_combine(ro[p], rl[p], is_lse_base_on_e=is_lse_base_on_e, out=out, out_lse=out_lse,
                                   timing=timing)


def reduce_scatter_merge(partial: torch.Tensor, lse: torch.Tensor, out=None, out_lse=None, timing=None):
    """Reduce-scatter flavour of the in-place merge for all N ranks at once.

    partial [N, T, H, D] and lse [N, T, H] hold every rank's partial result.
    Rank r owns heads [r*H/N, (r+1)*H/N) and merges them from all N partials
    without writing scaled partials back: the all-reduce followed by a head
    slice in the code excerpt of cp_lse_ag_out_rs_mha (sglang PR #34213
    report), done as a one-shot reduce-scatter.  After that exchange rank r
    holds its slice of every peer's partial contiguously and combines it.
    The N ranks' slices tile the H heads, so their combines together are one
    out-of-place combine over all heads of the stack, which reads every
    peer's partial front to back as each rank reads its received slice.
    Returns out [T, H, D] (rank r's slice at heads r*H/N...) and the global
    LSE [T, H]."""
    N, T, H, D = partial.shape
    assert H % N == 0 and tuple(lse.shape) == (N, T, H)
    if out is None:
        out = torch.empty((T, H, D), dtype=partial.dtype, device=partial.device)
    if out_lse is None:
        out_lse = torch.empty((T, H), dtype=torch.float32, device=partial.device)
    ops.dcp_lse_combine(partial, lse, is_lse_base_on_e=True, out=out, out_lse=out_lse, timing=timing)
    return out, out_lse
