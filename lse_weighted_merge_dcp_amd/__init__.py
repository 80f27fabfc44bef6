"""libdcpmerge: the decode-context-parallel (DCP) attention partial-merge path
for AMD Instinct MI355X (gfx950).

Hand-written HIP kernels behind a C ABI (include/dcpmerge.h) for the three
steps of the path -- the stride-driven pack of rank-local partials into
per-peer send layouts, the LSE-weighted unpack-combine, and the in-place
merge -- with a thin ctypes binding.  The shared library is loaded on first
use and every call fails loudly if it is missing.
"""
from ._lib import DcpError, DcpLaunchError
from .ops import cp_lse_combine_inplace, dcp_lse_combine, dcp_pack_a2a_send, interleaved_views, lse_pack_dim

__all__ = ["DcpError", "DcpLaunchError", "cp_lse_combine_inplace", "dcp_lse_combine", "dcp_pack_a2a_send",
           "interleaved_views", "lse_pack_dim"]
