"""Calls too large for one launch: more than 2^30 rows of one head each, which
the launchers split over several launches (every launch stays within 32-bit
indices and 2^23 workgroups), with byte offsets far beyond 4 GiB inside each
launch.  Rows are kept small (bf16, D = 8: 16-byte rows) so each case fits in
a few tens of GiB.  The tokens on both sides of every possible split point,
the first and last tokens and random tokens are checked against the oracle."""
import numpy as np
import pytest
import torch

from lse_weighted_merge_dcp_amd import ops, timing
from oracle import oracle as orc

from helpers import check_lse, check_out, check_scaled, decode, say, to_host

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
H_ROWS = 512                 # heads per token in every case below
TOKENS = (1 << 21) + 3       # TOKENS * H_ROWS > 2^30 rows
SPLIT = 1 << 18              # with 16-byte rows every split falls on a multiple of this many tokens


def randn(shape, seed, dtype=torch.bfloat16, scale=1.0):
    g = torch.Generator(device=DEV).manual_seed(seed)
    return torch.randn(shape, generator=g, device=DEV, dtype=dtype) * scale


def sample(n, seed, k=200):
    pts = {0, n - 1}
    for s in range(SPLIT, n, SPLIT):
        pts.update({s - 2, s - 1, s, s + 1})
    pts.update(np.random.default_rng(seed).integers(0, n, size=k).tolist())
    return torch.from_numpy(np.array(sorted(p for p in pts if 0 <= p < n))).to(DEV)


def test_pack_beyond_one_launch():
    N, H, D, B = 2, H_ROWS, 8, TOKENS
    Hpr = H // N
    say("pack beyond one launch", B, H, D)
    src = randn((B, H, D), 1)
    lse = randn((B, H), 2, torch.float32, 3.0)
    send = torch.empty((N, B, Hpr, D + 2), dtype=torch.bfloat16, device=DEV)
    pay, words = ops.interleaved_views(send, D)
    ops.dcp_pack_a2a_send(src, lse, pay, words)
    torch.cuda.synchronize()
    bs = sample(B, 3)
    got = to_host(send[:, bs], "bf16")
    want = np.zeros_like(got)
    wp, ww = orc.interleaved_views_np(want, D, "bf16")
    orc.pack(to_host(src[bs], "bf16"), lse[bs].cpu().numpy(), wp, ww, N)
    assert np.array_equal(got, want)
    # a timing request spans the whole call: first launch's start to last launch's end
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s, e = timing.Event(), timing.Event()
    a.record()
    ops.dcp_pack_a2a_send(src, lse, pay, words)
    b.record()
    ops.dcp_pack_a2a_send(src, lse, pay, words, timing=(s, e))
    torch.cuda.synchronize()
    whole, timed = a.elapsed_time(b) * 1e3, s.elapsed_us(e)
    say("whole call %.0f us, timed %.0f us" % (whole, timed))
    assert 0.7 * whole < timed < 1.3 * whole
    del src, lse, send, pay, words
    torch.cuda.empty_cache()


def test_combine_beyond_one_launch():
    N, Hpr, D, B = 2, H_ROWS, 8, TOKENS
    say("combine beyond one launch", B, Hpr, D)
    recv = randn((N, B, Hpr, D), 4)
    rl = randn((N, B, Hpr), 5, torch.float32, 3.0)
    out, g = ops.dcp_lse_combine(recv, rl, is_lse_base_on_e=True)
    torch.cuda.synchronize()
    bs = sample(B, 6)
    ref, gr, mag, _ = orc.combine(to_host(recv[:, bs], "bf16"), rl[:, bs].cpu().numpy(), "bf16", False)
    check_out(decode(to_host(out[bs], "bf16"), "bf16"), ref, mag, "bf16")
    check_lse(g[bs].cpu().numpy(), gr)
    del recv, rl, out, g
    torch.cuda.empty_cache()


def test_inplace_beyond_one_launch():
    N, H, D, T = 2, H_ROWS, 8, TOKENS
    h0, h1 = 100, 300
    say("inplace beyond one launch", T, H, D)
    part = randn((N, T, H, D), 7)
    lse = randn((N, T, H), 8, torch.float32, 3.0)
    ts = sample(T, 9)
    before = to_host(part[:, ts], "bf16")
    out, g = ops.cp_lse_combine_inplace(part, lse, h0=h0, h1=h1, return_lse=True)
    torch.cuda.synchronize()
    scaled, ref, gr, mag = orc.inplace(before, lse[:, ts].cpu().numpy(), "bf16", False, h0=h0, h1=h1)
    check_scaled(decode(to_host(part[:, ts], "bf16"), "bf16"), scaled, "bf16")
    check_out(decode(to_host(out[ts], "bf16"), "bf16"), ref, mag, "bf16")
    check_lse(g[ts].cpu().numpy(), gr)
    del part, lse, out, g
    torch.cuda.empty_cache()


def test_combine_beyond_one_launch_fp8():
    """The same split with an fp8 payload (D = 16: 16-byte rows), random
    codes including the two NaN codes (guarded to 0)."""
    N, Hpr, D, B = 2, H_ROWS, 16, TOKENS
    say("combine beyond one launch, fp8", B, Hpr, D)
    g8 = torch.Generator(device=DEV).manual_seed(10)
    codes = torch.randint(0, 256, (N, B, Hpr, D), generator=g8, device=DEV, dtype=torch.uint8)
    rl = randn((N, B, Hpr), 11, torch.float32, 3.0)
    out, g = ops.dcp_lse_combine(codes.view(torch.float8_e4m3fn), rl, is_lse_base_on_e=False)
    torch.cuda.synchronize()
    bs = sample(B, 12)
    ref, gr, mag, _ = orc.combine(codes[:, bs].cpu().numpy(), rl[:, bs].cpu().numpy(), "fp8", True)
    check_out(decode(out.view(torch.uint8)[bs].cpu().numpy(), "fp8"), ref, mag, "fp8")
    check_lse(g[bs].cpu().numpy(), gr)
    del codes, rl, out, g
    torch.cuda.empty_cache()
