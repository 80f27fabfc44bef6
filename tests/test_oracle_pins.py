"""Pins of the fp64 oracle against what the pages and the mathematics fix.

None of these re-types the oracle's formulas.  They check it against:
  * hand-derived worked examples (tests/golden/merge_cases.json);
  * a library logsumexp (torch, fp64 CPU) over every special-value combination;
  * brute-force softmax attention split over KV chunks (the merge must undo the split);
  * closed forms and invariants: N = 1 identity, neutral rank, equal LSEs give the
    mean, base equivalence, shift and permutation invariance, weights sum to one;
  * P1's own view/permute construction of both pack layouts, and hand-built bytes.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attn_bruteforce as bf
from oracle import oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _num(x):
    if isinstance(x, str):
        return {"nan": math.nan, "inf": math.inf, "-inf": -math.inf,
                "log2(3)": math.log2(3), "log2(5)": math.log2(5), "ln(2)": math.log(2)}[x]
    return float(x)


def _same(a, b, tol):
    if math.isnan(b):
        return math.isnan(a)
    if math.isinf(b):
        return a == b
    return abs(a - b) <= tol


# --------------------------------------------------------------------------
# hand-derived fixtures
# --------------------------------------------------------------------------
def test_golden_merge_cases():
    cases = json.load(open(os.path.join(GOLDEN, "merge_cases.json")))["cases"]
    for c in cases:
        lse = np.array([_num(x) for x in c["lse"]], np.float32)
        o = np.array([[_num(x) for x in row] for row in c["o"]], np.float32)
        N, D = o.shape
        out, g, _, _ = orc.combine(o.reshape(N, 1, 1, D), lse.reshape(N, 1, 1), "f32", c["base2"])
        assert _same(g[0, 0], _num(c["G"]), 1e-12), c["name"]
        want = [_num(x) for x in c["out"]]
        for got, w in zip(out[0, 0], want):
            assert _same(got, w, 1e-12), (c["name"], out[0, 0], want)


def test_golden_pack_layouts():
    fx = json.load(open(os.path.join(GOLDEN, "pack_layouts.json")))
    N, B, H, D = fx["N"], fx["B"], fx["H"], fx["D"]
    o = np.array([[[10.0 * h + d for d in range(D)] for h in range(H)]], np.float32)
    lse = np.array([[0.5 + h for h in range(H)]], np.float32)
    Hpr = H // N
    send = np.full((N, B, Hpr, D + 1), -7.0, np.float32)
    orc.pack(o, lse, send[..., :D], send[..., D], N)
    np.testing.assert_array_equal(send.ravel(), np.array(fx["interleaved_words"], np.float32))
    part = np.full((B, Hpr, N, D), -7.0, np.float32)
    stats = np.full((B, Hpr, N, 2), 99.0, np.float32)
    orc.pack(o, lse, part.transpose(2, 0, 1, 3), stats[..., 0].transpose(2, 0, 1), N)
    np.testing.assert_array_equal(part.ravel(), np.array(fx["split_partial_o"], np.float32))
    np.testing.assert_array_equal(stats.ravel(), np.array(fx["split_stats"], np.float32))


# --------------------------------------------------------------------------
# global LSE against a library logsumexp, every special-value combination
# --------------------------------------------------------------------------
SPECIALS = [math.nan, math.inf, -math.inf, -1.25, 0.0, 2.5]


@pytest.mark.parametrize("base2", [False, True])
def test_global_lse_matches_library_logsumexp(base2):
    rows = list(itertools.product(SPECIALS, repeat=3))
    l = np.array(rows, np.float32).T.copy()                 # [3, rows]
    N, R = l.shape
    o = np.ones((N, R, 1, 1), np.float32)
    _, g, _, w = orc.combine(o, l.reshape(N, R, 1), "f32", base2)
    lt = torch.tensor(l.astype(np.float64))
    if base2:
        ref = torch.logsumexp(lt * math.log(2.0), dim=0) / math.log(2.0)
    else:
        ref = torch.logsumexp(lt, dim=0)
    for r in range(R):
        assert _same(g[r, 0], float(ref[r]), 1e-12), (rows[r], g[r, 0], float(ref[r]))
    # weights: library exp of (l - G), guarded; sum to 1 whenever G is finite
    for r in range(R):
        G = float(ref[r])
        for i in range(N):
            x = (2.0 ** (float(l[i, r]) - G)) if base2 else math.exp(float(l[i, r]) - G) \
                if not (math.isnan(G) or math.isnan(l[i, r])) else math.nan
            want = x if math.isfinite(x) else 0.0
            assert abs(w[i, r, 0] - want) <= 1e-12
        if math.isfinite(G):
            assert abs(w[:, r, 0].sum() - 1.0) <= 1e-12


def test_random_lse_matches_library():
    rng = np.random.default_rng(5)
    for N in (1, 2, 3, 8, 16, 17, 40):
        l = rng.normal(0, 6, size=(N, 50)).astype(np.float32)
        o = rng.normal(size=(N, 50, 1, 4)).astype(np.float32)
        _, g, _, _ = orc.combine(o, l.reshape(N, 50, 1), "f32", False)
        ref = torch.logsumexp(torch.tensor(l.astype(np.float64)), dim=0).numpy()
        np.testing.assert_allclose(g[:, 0], ref, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# brute force: merging per-slice attention reproduces unsplit attention
# --------------------------------------------------------------------------
@pytest.mark.parametrize("base2", [False, True])
@pytest.mark.parametrize("N,L,split", [(2, 17, "rr"), (4, 37, "rr"), (8, 5, "rr"), (3, 40, "contig"),
                                       (16, 100, "rr"), (5, 0, "rr"), (1, 9, "rr"), (17, 60, "contig")])
def test_split_attention_bruteforce(base2, N, L, split):
    rng = np.random.default_rng(100 + N * 7 + L)
    H, dk, D = 6, 16, 24
    q = rng.normal(size=(H, dk))
    K = rng.normal(size=(L, dk)) * 1.5
    V = rng.normal(size=(L, D))
    scale = 1.0 / math.sqrt(dk)
    owner = bf.round_robin_owner(L, N) if split == "rr" else bf.contiguous_owner(L, N)
    outs, lses = bf.split_partials(q, K, V, scale, owner, N)
    full_o, full_l = bf.attention(q, K, V, scale)
    if base2:
        lses = lses * math.log2(math.e)
        full_l = full_l * math.log2(math.e)
    # the oracle takes its inputs in the payload type; use fp32 values carried exactly in fp64
    o32 = outs.astype(np.float32)
    l32 = lses.astype(np.float32)
    out, g, _, _ = orc.combine(o32.reshape(N, 1, H, D), l32.reshape(N, 1, H), "f32", base2)
    # reference: attention of the same fp32-rounded partials is within fp32 rounding of the full result
    np.testing.assert_allclose(out[0], full_o, rtol=0, atol=2e-6 * max(1.0, np.abs(full_o).max()))
    if L == 0:
        assert np.all(np.isneginf(g))
    else:
        np.testing.assert_allclose(g[0], full_l, rtol=0, atol=4e-6 * max(1.0, np.abs(full_l).max()))


def test_split_attention_exact_in_fp64():
    """With no fp32 rounding of the partials the merge is exact to fp64 rounding."""
    rng = np.random.default_rng(7)
    H, dk, D, L, N = 4, 8, 10, 29, 4
    q = rng.normal(size=(H, dk))
    K = rng.normal(size=(L, dk))
    V = rng.normal(size=(L, D))
    outs, lses = bf.split_partials(q, K, V, 0.4, bf.round_robin_owner(L, N), N)
    full_o, full_l = bf.attention(q, K, V, 0.4)
    # evaluate the merge in fp64 by calling the C routine directly on fp64 inputs
    lib = orc._load()
    rows = H
    o = np.ascontiguousarray(outs.reshape(N, rows, D))
    l = np.ascontiguousarray(lses.reshape(N, rows))
    out = np.empty((rows, D)); g = np.empty(rows); mag = np.empty((rows, D)); w = np.empty((N, rows))
    lib.orc_combine(orc._ptr(o), orc._ptr(l), N, rows, D, 0, orc._ptr(out), orc._ptr(g), orc._ptr(mag), orc._ptr(w))
    np.testing.assert_allclose(out, full_o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(g, full_l, rtol=1e-13, atol=0)


# --------------------------------------------------------------------------
# closed forms and invariants
# --------------------------------------------------------------------------
def _rand(N, rows, D, seed, sd=3.0):
    rng = np.random.default_rng(seed)
    o = rng.normal(size=(N, rows, 1, D)).astype(np.float32)
    l = rng.normal(0, sd, size=(N, rows, 1)).astype(np.float32)
    return o, l


def test_n1_identity_bits():
    o, l = _rand(1, 8, 5, 1)
    o[0, 0, 0, 0] = np.nan
    o[0, 1, 0, 1] = np.inf
    l[0, 2, 0] = np.nan
    out, g, _, _ = orc.combine(o, l, "f32", False)
    np.testing.assert_array_equal(out.astype(np.float32).view(np.uint32), o[0].view(np.uint32))
    np.testing.assert_array_equal(g.astype(np.float32).view(np.uint32), l[0].view(np.uint32))


@pytest.mark.parametrize("base2", [False, True])
def test_neutral_rank_changes_nothing(base2):
    o, l = _rand(5, 30, 7, 2)
    out, g, _, _ = orc.combine(o, l, "f32", base2)
    o2 = np.concatenate([o[:2], np.zeros_like(o[:1]), o[2:]])
    l2 = np.concatenate([l[:2], np.full_like(l[:1], -np.inf), l[2:]])
    out2, g2, _, _ = orc.combine(o2, l2, "f32", base2)
    np.testing.assert_array_equal(out, out2)
    np.testing.assert_array_equal(g, g2)


def test_all_neutral_gives_zero_and_minus_inf():
    o = np.zeros((4, 3, 1, 5), np.float32)
    l = np.full((4, 3, 1), -np.inf, np.float32)
    out, g, _, _ = orc.combine(o, l, "f32", True)
    assert np.all(out == 0) and np.all(np.isneginf(g))


@pytest.mark.parametrize("base2", [False, True])
def test_equal_lse_gives_mean(base2):
    o, _ = _rand(6, 20, 9, 3)
    c = np.float32(1.75)
    l = np.full((6, 20, 1), c, np.float32)
    out, g, _, _ = orc.combine(o, l, "f32", base2)
    np.testing.assert_allclose(out[:, 0], o.astype(np.float64).mean(axis=0)[:, 0], rtol=0, atol=1e-14)
    want_g = float(c) + (math.log2(6) if base2 else math.log(6))
    np.testing.assert_allclose(g, want_g, rtol=0, atol=1e-14)


def test_base_equivalence():
    o, l = _rand(8, 40, 6, 4, sd=2.0)
    out_e, g_e, _, _ = orc.combine(o, l, "f32", False)
    # base-2 LSEs of the same partials: l * log2(e); use fp64 to avoid rounding the LSE twice
    lib = orc._load()
    N, rows, D = 8, 40, 6
    oo = np.ascontiguousarray(o.astype(np.float64).reshape(N, rows, D))
    l2 = np.ascontiguousarray(l.astype(np.float64).reshape(N, rows) * math.log2(math.e))
    out2 = np.empty((rows, D)); g2 = np.empty(rows); mag = np.empty((rows, D)); w = np.empty((N, rows))
    lib.orc_combine(orc._ptr(oo), orc._ptr(l2), N, rows, D, 1, orc._ptr(out2), orc._ptr(g2), orc._ptr(mag), orc._ptr(w))
    np.testing.assert_allclose(out2, out_e[:, 0], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(g2, g_e[:, 0] * math.log2(math.e), rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("base2", [False, True])
def test_shift_and_permutation_invariance(base2):
    o, l = _rand(7, 25, 4, 6)
    l = (np.round(l * 1024) / 1024).astype(np.float32)   # on a 2^-10 grid, so l + c is exact in fp32
    out, g, _, _ = orc.combine(o, l, "f32", base2)
    c = np.float32(12.5)
    out_s, g_s, _, _ = orc.combine(o, l + c, "f32", base2)
    np.testing.assert_allclose(out_s, out, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(g_s, g + float(c), rtol=0, atol=1e-12)
    perm = np.random.default_rng(1).permutation(7)
    out_p, g_p, _, _ = orc.combine(o[perm], l[perm], "f32", base2)
    np.testing.assert_allclose(out_p, out, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(g_p, g, rtol=0, atol=1e-13)


def test_guards_match_zeroed_partials():
    """nan_to_num on o: a non-finite element contributes exactly like a 0."""
    o, l = _rand(4, 12, 6, 8)
    o_bad = o.copy()
    o_bad[1, 3, 0, 2] = np.nan
    o_bad[2, 5, 0, 0] = np.inf
    o_bad[0, 7, 0, 5] = -np.inf
    o_zero = np.where(np.isfinite(o_bad), o_bad, 0).astype(np.float32)
    a, ga, _, _ = orc.combine(o_bad, l, "f32", False)
    b, gb, _, _ = orc.combine(o_zero, l, "f32", False)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(ga, gb)


def test_decoders_exact():
    rng = np.random.default_rng(9)
    x = rng.normal(size=1000).astype(np.float32)
    h = x.astype(np.float16)
    np.testing.assert_array_equal(orc.to_f64(h, "f16"), h.astype(np.float64))
    bf = torch.tensor(x).to(torch.bfloat16)
    bits = bf.view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(orc.to_f64(bits, "bf16"), bf.to(torch.float64).numpy())


def test_fp8_decoder_against_torch_and_hand_values():
    """OCP FP8 E4M3: every one of the 256 codes decodes as torch's
    float8_e4m3fn does (NaN where torch has NaN), and a few codes worked by
    hand from the format: 0x38 = 1, 0x7E = 448 (largest), 0x08 = 2^-6
    (smallest normal), 0x01 = 2^-9 (smallest subnormal), 0x80 = -0, 0xFE =
    -448, 0x70 = 2^(14-7) = 128, 0x7F and 0xFF NaN."""
    codes = np.arange(256, dtype=np.uint8)
    got = orc.to_f64(codes, "fp8")
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(np.isnan(got), np.isnan(want))
    np.testing.assert_array_equal(got[~np.isnan(got)], want[~np.isnan(want)])
    hand = {0x38: 1.0, 0x7E: 448.0, 0x08: 2.0 ** -6, 0x01: 2.0 ** -9, 0x00: 0.0, 0xFE: -448.0,
            0x70: 128.0, 0x3C: 1.5, 0xB8: -1.0, 0x07: 7 * 2.0 ** -9}
    for c, v in hand.items():
        assert got[c] == v, hex(c)
    assert math.copysign(1.0, got[0x80]) == -1.0 and got[0x80] == 0.0
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF])
    assert np.isnan(got).sum() == 2 and not np.isinf(got).any()


# --------------------------------------------------------------------------
# in-place merge: consistent with the combine, the brute force and the slice
# --------------------------------------------------------------------------
@pytest.mark.parametrize("base2", [False, True])
def test_inplace_matches_split_attention(base2):
    rng = np.random.default_rng(11)
    N, H, dk, D, L, T = 4, 8, 8, 12, 23, 3
    partial = np.empty((N, T, H, D), np.float64)
    lse = np.empty((N, T, H), np.float64)
    full_o = np.empty((T, H, D)); full_l = np.empty((T, H))
    for t in range(T):
        q = rng.normal(size=(H, dk)); K = rng.normal(size=(L + t, dk)); V = rng.normal(size=(L + t, D))
        o, l = bf.split_partials(q, K, V, 0.3, bf.round_robin_owner(L + t, N), N)
        partial[:, t] = o; lse[:, t] = l
        full_o[t], full_l[t] = bf.attention(q, K, V, 0.3)
    if base2:
        lse = lse * math.log2(math.e); full_l = full_l * math.log2(math.e)
    p32 = partial.astype(np.float32); l32 = lse.astype(np.float32)
    scaled, out, g, _ = orc.inplace(p32, l32, "f32", base2)
    np.testing.assert_allclose(out, full_o, rtol=0, atol=3e-6)
    np.testing.assert_allclose(g, full_l, rtol=0, atol=3e-6)
    np.testing.assert_allclose(scaled.sum(axis=0), out, rtol=1e-12, atol=1e-14)
    # the head slice [h0, h1) of one rank is the same numbers
    _, out_s, g_s, _ = orc.inplace(p32, l32, "f32", base2, h0=2, h1=4)
    np.testing.assert_array_equal(out_s, out[:, 2:4]); np.testing.assert_array_equal(g_s, g[:, 2:4])


def test_inplace_partial_ranks_sum_to_full():
    """Holding only some ranks' partials (rank0, P) gives that rank subset's share."""
    o, l = _rand(6, 10, 5, 12)
    part = o.reshape(6, 10, 1, 5)
    lse = l.reshape(6, 10, 1)
    _, full, g, _ = orc.inplace(part, lse, "f32", False)
    acc = np.zeros_like(full)
    for r0, P in ((0, 2), (2, 3), (5, 1)):
        sc, out, g2, _ = orc.inplace(part[r0:r0 + P], lse, "f32", False, rank0=r0)
        acc += out
        np.testing.assert_array_equal(g2, g)
    np.testing.assert_allclose(acc, full, rtol=1e-12, atol=1e-14)


def test_inplace_scaled_equals_weight_times_guarded():
    o, l = _rand(3, 9, 4, 13)
    o[1, 2, 0, 1] = np.nan
    l[2, 4, 0] = np.inf
    scaled, out, g, _ = orc.inplace(o, l, "f32", False)
    _, gc, _, w = orc.combine(o, l, "f32", False)
    og = np.where(np.isfinite(o), o, 0).astype(np.float64)
    np.testing.assert_array_equal(scaled, og * w[..., None])
    np.testing.assert_array_equal(g, gc)
    # the +inf row: every weight is 0, so the merged row and its scaled partials are 0
    assert np.all(scaled[:, 4] == 0) and np.isposinf(g[4, 0])


def test_inplace_n1_untouched():
    o, l = _rand(1, 6, 3, 14)
    o[0, 1, 0, 1] = np.nan
    scaled, out, g, _ = orc.inplace(o, l, "f32", False)
    np.testing.assert_array_equal(scaled.astype(np.float32).view(np.uint32), o.view(np.uint32))


# --------------------------------------------------------------------------
# pack against the page's own construction (view + permute) and round trip
# --------------------------------------------------------------------------
@pytest.mark.parametrize("N,B,Hpr,D", [(2, 4, 8, 128), (4, 1, 16, 512), (2, 3, 1, 5), (8, 2, 4, 64)])
def test_pack_split_layout_matches_page_construction(N, B, Hpr, D):
    """sglang PR #34651 report, split-layout test excerpt: expected partial_o is
    out.view(B,N,Hpr,D).permute(0,2,1,3), expected stats slot 0 is
    lse.view(B,N,Hpr).permute(0,2,1); slot 1 keeps its bytes."""
    H = N * Hpr
    g = torch.Generator().manual_seed(N * 100 + B)
    out = torch.randn(B, H, D, generator=g).to(torch.bfloat16)
    lse = torch.randn(B, H, generator=g)
    o_np = out.view(torch.int16).numpy().view(np.uint16)
    l_np = lse.numpy()
    rng = np.random.default_rng(3)
    part = np.frombuffer(rng.bytes(B * Hpr * N * D * 2), np.uint16).reshape(B, Hpr, N, D).copy()
    stats = np.frombuffer(rng.bytes(B * Hpr * N * 2 * 4), np.float32).reshape(B, Hpr, N, 2).copy()
    slot1 = stats[..., 1].copy()
    orc.pack(o_np, l_np, part.transpose(2, 0, 1, 3), stats[..., 0].transpose(2, 0, 1), N)
    want_o = out.view(B, N, Hpr, D).permute(0, 2, 1, 3).contiguous().view(torch.int16).numpy().view(np.uint8)
    want_l = lse.view(B, N, Hpr).permute(0, 2, 1).contiguous().numpy()
    np.testing.assert_array_equal(part.view(np.uint8).reshape(-1), want_o.reshape(-1))
    np.testing.assert_array_equal(stats[..., 0].view(np.uint32), want_l.view(np.uint32))
    np.testing.assert_array_equal(stats[..., 1].view(np.uint32), slot1.view(np.uint32))


@pytest.mark.parametrize("dt,N,B,Hpr,D", [("bf16", 8, 3, 16, 512), ("f32", 2, 4, 4, 64), ("f16", 4, 5, 3, 10)])
def test_pack_interleaved_matches_page_construction(dt, N, B, Hpr, D):
    """Peer-outer interleaved send buffer [N,B,Hpr,D+lpd]: payload slot = the
    page's out.view(B,N,Hpr,D) moved to peer-outer order; LSE = fp32 word D/lpd."""
    H = N * Hpr
    g = torch.Generator().manual_seed(7)
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32, "f16": torch.float16}[dt]
    out = torch.randn(B, H, D, generator=g).to(tdt)
    lse = torch.randn(B, H, generator=g) * 4
    npdt = {"bf16": np.uint16, "f32": np.float32, "f16": np.float16}[dt]
    o_np = out.view(torch.int16).numpy().view(np.uint16) if dt == "bf16" else out.numpy()
    lpd = 4 // orc.ESIZE[dt]
    send = np.frombuffer(np.random.default_rng(1).bytes(N * B * Hpr * (D + lpd) * orc.ESIZE[dt]), npdt)
    send = send.reshape(N, B, Hpr, D + lpd).copy()
    pay, words = orc.interleaved_views_np(send, D, dt)
    orc.pack(o_np, lse.numpy(), pay, words, N)
    want = out.view(B, N, Hpr, D).permute(1, 0, 2, 3).contiguous()
    want_bytes = (want.view(torch.int16) if dt == "bf16" else want).numpy().view(np.uint8)
    np.testing.assert_array_equal(np.ascontiguousarray(pay).view(np.uint8).reshape(-1), want_bytes.reshape(-1))
    want_l = lse.view(B, N, Hpr).permute(1, 0, 2).contiguous().numpy()
    np.testing.assert_array_equal(np.ascontiguousarray(words).view(np.uint32), want_l.view(np.uint32))


def test_pack_round_trip_through_exchange():
    """After the all-to-all, destination r holds recv[src, b, hl] = out_src[b, r*Hpr + hl]."""
    N, B, Hpr, D = 4, 3, 2, 6
    H = N * Hpr
    rng = np.random.default_rng(21)
    outs = rng.normal(size=(N, B, H, D)).astype(np.float32)
    lses = rng.normal(size=(N, B, H)).astype(np.float32)
    send = np.zeros((N, N, B, Hpr, D + 1), np.float32)        # [src, peer, B, Hpr, D+1]
    for s in range(N):
        orc.pack(outs[s], lses[s], send[s, ..., :D], send[s, ..., D], N)
    for r in range(N):
        recv = send[:, r]                                       # the exchange: chunk r of every source
        for s in range(N):
            np.testing.assert_array_equal(recv[s, ..., :D], outs[s][:, r * Hpr:(r + 1) * Hpr])
            np.testing.assert_array_equal(recv[s, ..., D], lses[s][:, r * Hpr:(r + 1) * Hpr])


@pytest.mark.parametrize("dt", ["bf16", "f32", "f16"])
def test_pack_zero_kv_tokens_become_neutral(dt):
    """A token for which this rank owns no KV is sent as the neutral pair
    (0, -inf): the same bytes as packing an output row of zeros and an LSE of
    -inf (sglang PR #33926 report, 实现拆解 item 3, fixup_zero_kv_rows)."""
    N, B, Hpr, D = 4, 6, 3, 40
    H = N * Hpr
    g = torch.Generator().manual_seed(3)
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32, "f16": torch.float16}[dt]
    out = torch.randn(B, H, D, generator=g).to(tdt)
    lse = torch.randn(B, H, generator=g)
    kv = np.array([5, 0, 1, 0, 0, 9], np.int32)
    o_np = out.view(torch.int16).numpy().view(np.uint16) if dt == "bf16" else out.numpy()
    neutral_o = o_np.copy()
    neutral_l = lse.numpy().copy()
    neutral_o[kv == 0] = 0
    neutral_l[kv == 0] = -np.inf
    lpd = 4 // orc.ESIZE[dt]
    npdt = {"bf16": np.uint16, "f32": np.float32, "f16": np.float16}[dt]
    a = np.zeros((N, B, Hpr, D + lpd), npdt)
    b = np.zeros((N, B, Hpr, D + lpd), npdt)
    pa, wa = orc.interleaved_views_np(a, D, dt)
    pb, wb = orc.interleaved_views_np(b, D, dt)
    orc.pack(o_np, lse.numpy(), pa, wa, N, kv_len=kv)
    orc.pack(neutral_o, neutral_l, pb, wb, N)
    np.testing.assert_array_equal(a.view(np.uint8), b.view(np.uint8))
    assert np.all(np.isneginf(wa[:, 1])) and np.all(wa[:, 0] == lse.numpy().reshape(B, N, Hpr).transpose(1, 0, 2)[:, 0])



def test_fp8_worked_example():
    """Two fp8 peers merged by the oracle, worked by hand.  Codes: peer 0 =
    (0x38, 0x7E, 0x01, 0x7F) = (1, 448, 2^-9, NaN), peer 1 = (0x3C, 0xFE,
    0x00, 0x40) = (1.5, -448, 0, 2).  Equal LSEs weigh each by 1/2: out =
    (1.25, 0, 2^-10, 1) (the NaN partial counts as 0).  LSEs (0, ln 3) weigh
    them 1/4 and 3/4: out = (1.375, -224, 2^-11, 1.5), and G = ln 4."""
    o = np.array([[0x38, 0x7E, 0x01, 0x7F], [0x3C, 0xFE, 0x00, 0x40]], np.uint8).reshape(2, 1, 1, 4)
    out, g, _, _ = orc.combine(o, np.zeros((2, 1, 1), np.float32), "fp8", False)
    np.testing.assert_array_equal(out.reshape(-1), [1.25, 0.0, 2.0 ** -10, 1.0])
    assert abs(g.item() - math.log(2.0)) < 1e-15
    # ln 3 rounded to fp32 moves the weights off 1/4 and 3/4 by about 1e-8
    lse = np.array([0.0, math.log(3.0)], np.float32).reshape(2, 1, 1)
    out, g, _, _ = orc.combine(o, lse, "fp8", False)
    np.testing.assert_allclose(out.reshape(-1), [1.375, -224.0, 2.0 ** -11, 1.5], rtol=1e-7, atol=0)
    assert abs(g.item() - math.log(4.0)) < 1e-7
