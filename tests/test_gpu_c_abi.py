"""The C ABI used from plain C (tests/c_abi_client.c: gcc, the HIP runtime
and libdcpmerge.so, no Python or torch in the process): pack of every rank
into interleaved send buffers, then the combine of every destination through
transposed strides.  The send buffers must equal the oracle's byte for byte,
the merged rows and global LSEs must be within the stated tolerance."""
import os
import subprocess

import numpy as np
import pytest
import torch

from lse_weighted_merge_dcp_amd import synth
from oracle import oracle as orc

from helpers import NP_DT, check_lse, check_out, decode, say

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLIENT = os.path.join(ROOT, "tests", "c_abi_client")
DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2, "fp8": 3}


@pytest.mark.parametrize("dt,N,B,H,D,base2", [
    ("f32", 2, 4, 8, 64, False),       # row pack, short-row combine
    ("bf16", 8, 3, 32, 512, True),     # flat-stream pack, row-per-wave combine
    ("f16", 4, 5, 12, 128, False),     # row pack, short-row combine, 3 heads per rank
    ("fp8", 8, 3, 32, 512, True),      # fp8: stream pack (two LSE words in most wave-steps), one-row-per-wave combine
])
def test_c_client_pack_and_combine(tmp_path, dt, N, B, H, D, base2):
    assert os.path.exists(CLIENT), "tests/c_abi_client is not built: run __graft_entry__.build()"
    say("c client", dt, N, B, H, D, base2)
    g = torch.Generator().manual_seed(N * 100 + D)
    out = synth.to_storage(torch.randn(N, B, H, D, generator=g), dt)
    lse = np.random.default_rng(D + B).normal(0, 3, size=(N, B, H)).astype(np.float32)
    lse[0, 0, 0] = -np.inf
    lse[:, 1, 1] = -np.inf
    (tmp_path / "meta.txt").write_text("%d %d %d %d %d %d\n" % (N, B, H, D, DTYPE_CODE[dt], 1 if base2 else 0))
    np.ascontiguousarray(out).tofile(tmp_path / "out.bin")
    lse.tofile(tmp_path / "lse.bin")

    r = subprocess.run([CLIENT, str(tmp_path)], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stderr
    assert "rejected call: DCP_ERR_NULL" in r.stdout
    assert "timed combine: " in r.stdout

    lpd = 4 // np.dtype(NP_DT[dt]).itemsize
    Hpr = H // N
    send = np.fromfile(tmp_path / "send.bin", NP_DT[dt]).reshape(N, N, B, Hpr, D + lpd)
    want = np.zeros_like(send)
    pay, words = orc.interleaved_views_np(want, D, dt)
    for s in range(N):
        orc.pack(out[s], lse[s], pay[s], words[s], N)
    assert np.array_equal(send.view(np.uint8), want.view(np.uint8))

    comb = np.fromfile(tmp_path / "comb.bin", NP_DT[dt]).reshape(N, B, Hpr, D)
    gl = np.fromfile(tmp_path / "g.bin", np.float32).reshape(N, B, Hpr)
    for p in range(N):
        ref, gr, mag, _ = orc.combine(pay[:, p], words[:, p], dt, base2)
        check_out(decode(comb[p], dt), ref, mag, dt, "dst %d" % p)
        check_lse(gl[p], gr)
