"""Zero-KV neutralisation fused into the pack (sglang PR #33926 report,
实现拆解 item 3: a rank that owns no part of a token's KV emits the neutral
pair (0, -inf)), on the GPU against the oracle.

* bit-exact pack with kv_len on the interleaved (stream and row kernels) and
  split layouts;
* end to end: round-robin KV ownership with sequences shorter than N leaves
  some ranks empty; their attention outputs are garbage (NaN, huge values),
  the pack neutralises them, and the merge reproduces unsplit attention.
"""
import math

import numpy as np
import pytest
import torch

from lse_weighted_merge_dcp_amd import ops, sim, synth
from oracle import attn_bruteforce as bf
from oracle import oracle as orc

from helpers import NP_DT, TORCH_DT, say, to_dev, to_host

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.mark.parametrize("dt,N,B,Hpr,D,layout", [
    ("bf16", 8, 9, 16, 512, "interleaved"),   # stream kernel, 4-wave workgroups
    ("bf16", 16, 40, 8, 512, "interleaved"),  # stream kernel, 8-wave workgroups (>= 32768 wave-steps)
    ("bf16", 16, 64, 8, 512, "interleaved"),  # stream kernel, XCD-chunked 4-wave workgroups (>= 131072 wave-steps)
    ("bf16", 16, 50, 8, 512, "interleaved"),  # 8-wave launch with nontemporal loads (100 MiB of source)
    ("fp8", 16, 128, 8, 512, "interleaved"),  # the same launch with two LSE words per wave-step
    ("f32", 2, 7, 4, 64, "interleaved"),      # row kernel (short rows)
    ("f16", 4, 6, 16, 128, "split"),          # split layout
    ("fp8", 8, 9, 16, 512, "interleaved"),    # fp8: stream kernel, 516-byte rows (two LSE words in most wave-steps)
    ("fp8", 4, 6, 16, 128, "split"),          # fp8 split layout
])
def test_pack_neutralises_zero_kv_tokens(dt, N, B, Hpr, D, layout):
    say("pack kv_len", dt, N, B, Hpr, D, layout)
    H = N * Hpr
    g = torch.Generator().manual_seed(B * 11 + D)
    out = synth.to_storage(torch.randn(N, B, H, D, generator=g), dt)
    lse = np.random.default_rng(D).normal(0, 3, size=(N, B, H)).astype(np.float32)
    kv = np.random.default_rng(B).integers(0, 3, size=(N, B)).astype(np.int32)   # about a third are 0
    kv[0, 0], kv[N - 1, B - 1] = 0, 0
    o_d, l_d, kv_d = to_dev(out, dt, DEV), torch.from_numpy(lse).to(DEV), torch.from_numpy(kv).to(DEV)
    esz = np.dtype(NP_DT[dt]).itemsize
    if layout == "interleaved":
        st = sim.StackedInterleaved(N, B, H, D, TORCH_DT[dt], DEV)
        fill = np.frombuffer(np.random.default_rng(5).bytes(st.send.numel() * esz), NP_DT[dt]).reshape(st.send.shape).copy()
        st.send.copy_(to_dev(fill, dt, DEV))
        st.pack(o_d, l_d, kv_len=kv_d)
        host = fill.copy()
        hp, hw = orc.interleaved_views_np(host, D, dt)
        for r in range(N):
            orc.pack(out[r], lse[r], hp[r], hw[r], N, kv_len=kv[r])
        assert np.array_equal(to_host(st.send, dt).view(np.uint8), host.view(np.uint8))
    else:
        st = sim.StackedSplit(N, B, H, D, TORCH_DT[dt], DEV)
        pf = np.frombuffer(np.random.default_rng(6).bytes(st.partial_o.numel() * esz), NP_DT[dt]).reshape(st.partial_o.shape).copy()
        sf = np.frombuffer(np.random.default_rng(7).bytes(st.stats.numel() * 4), np.float32).reshape(st.stats.shape).copy()
        st.partial_o.copy_(to_dev(pf, dt, DEV))
        st.stats.copy_(torch.from_numpy(sf.copy()).to(DEV))
        st.pack(o_d, l_d, kv_len=kv_d)
        hp, hs = pf.copy(), sf.copy()
        for r in range(N):
            orc.pack(out[r], lse[r], hp[r].transpose(2, 0, 1, 3), hs[r][..., 0].transpose(2, 0, 1), N, kv_len=kv[r])
        assert np.array_equal(to_host(st.partial_o, dt).view(np.uint8), hp.view(np.uint8))
        assert np.array_equal(st.stats.cpu().numpy().view(np.uint32), hs.view(np.uint32))


@pytest.mark.parametrize("base2", [False, True])
def test_empty_ranks_neutralised_end_to_end(base2):
    """N = 8 ranks, round-robin KV ownership; tokens with sequences of 1..20
    keys leave some ranks with nothing.  Those ranks' partial outputs are
    garbage; with kv_len the pack sends (0, -inf) for them and the merged
    result is unsplit attention."""
    N, H, dk, D = 8, 16, 16, 64
    Hpr = H // N
    lens = [1, 3, 5, 8, 13, 20]
    B = len(lens)
    rng = np.random.default_rng(17)
    outs = np.zeros((N, B, H, D), np.float32)
    lses = np.zeros((N, B, H), np.float32)
    kv = np.zeros((N, B), np.int32)
    full_o = np.zeros((B, H, D))
    full_l = np.zeros((B, H))
    for b, L in enumerate(lens):
        q = rng.normal(size=(H, dk))
        K = rng.normal(size=(L, dk))
        V = rng.normal(size=(L, D))
        owner = bf.round_robin_owner(L, N)
        po, pl = bf.split_partials(q, K, V, 0.25, owner, N)
        full_o[b], full_l[b] = bf.attention(q, K, V, 0.25)
        for r in range(N):
            kv[r, b] = int(synth.dcp_local_len(np.array([L]), N, r)[0])
            if kv[r, b] == 0:
                outs[r, b] = np.nan if (r + b) % 2 else 3e38   # whatever an attention kernel left there
                lses[r, b] = 7.0 if (r + b) % 3 else np.nan
            else:
                outs[r, b] = po[r]
                lses[r, b] = pl[r] * (math.log2(math.e) if base2 else 1.0)
    if base2:
        full_l = full_l * math.log2(math.e)
    assert (kv == 0).any() and (kv > 0).any()
    st = sim.StackedInterleaved(N, B, H, D, torch.float32, DEV)
    st.pack(torch.from_numpy(outs).to(DEV), torch.from_numpy(lses).to(DEV), kv_len=torch.from_numpy(kv).to(DEV))
    out, g = st.combine(is_lse_base_on_e=not base2)
    got = out.cpu().numpy()        # [dst, B, Hpr, D]
    gl = g.cpu().numpy()
    for p in range(N):
        np.testing.assert_allclose(got[p], full_o[:, p * Hpr:(p + 1) * Hpr], rtol=0, atol=2e-6)
        np.testing.assert_allclose(gl[p], full_l[:, p * Hpr:(p + 1) * Hpr], rtol=0, atol=1e-5)
