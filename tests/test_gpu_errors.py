"""A stale HIP error left on the calling thread by an unrelated call does not
make a library call fail: each launch's own status is checked, not the
thread's last error."""
import ctypes

import numpy as np
import pytest
import torch

from lse_weighted_merge_dcp_amd import ops
from oracle import oracle as orc

from helpers import check_lse, check_out, say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def loaded_hip_runtime():
    """The HIP runtime this process already uses (same path, same instance)."""
    for line in open("/proc/self/maps"):
        if "libamdhip64.so" in line:
            lib = ctypes.CDLL(line.split()[-1])
            lib.hipSetDevice.argtypes = [ctypes.c_int]
            lib.hipSetDevice.restype = ctypes.c_int
            lib.hipGetLastError.restype = ctypes.c_int
            return lib
    raise RuntimeError("libamdhip64 is not loaded")


def test_stale_error_does_not_fail_a_call():
    say("stale error")
    N, B, H, D = 2, 3, 4, 64
    rng = np.random.default_rng(3)
    out = rng.normal(size=(B, H, D)).astype(np.float32)
    lse = rng.normal(0, 2, size=(B, H)).astype(np.float32)
    d_out, d_lse = torch.from_numpy(out).to(DEV), torch.from_numpy(lse).to(DEV)
    send = torch.zeros((N, B, H // N, D + 1), device=DEV)
    pay, words = ops.interleaved_views(send, D)
    comb = torch.empty((B, H // N, D), device=DEV)
    g = torch.empty((B, H // N), device=DEV)
    torch.cuda.synchronize()
    hip = loaded_hip_runtime()
    assert hip.hipSetDevice(123456) != 0          # an invalid device: leaves an error on this thread
    try:
        ops.dcp_pack_a2a_send(d_out, d_lse, pay, words)
        ops.dcp_lse_combine(pay, words, is_lse_base_on_e=True, out=comb, out_lse=g)
    finally:
        hip.hipGetLastError()                     # leave the thread clean for what follows
    torch.cuda.synchronize()
    want = np.zeros((N, B, H // N, D + 1), np.float32)
    wp, ww = orc.interleaved_views_np(want, D, "f32")
    orc.pack(out, lse, wp, ww, N)
    assert np.array_equal(send.cpu().numpy().view(np.uint32), want.view(np.uint32))
    ref, gr, mag, _ = orc.combine(wp, ww, "f32", False)
    check_out(comb.cpu().numpy(), ref, mag, "f32")
    check_lse(g.cpu().numpy(), gr)
