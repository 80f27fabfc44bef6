"""GPU parity of dcp_unpack_combine against the fp64 oracle.

Inputs of the combine tests are receive buffers built on the host by the
oracle's own pack (so no input comes from the HIP path) and uploaded; the
end-to-end tests run the HIP pack, the simulated exchange (views) and the HIP
combine, and compare with the oracle's pack -> exchange -> combine.
"""
import itertools
import math

import numpy as np
import pytest
import torch

from lse_weighted_merge_dcp_amd import ops, sim, synth
from oracle import oracle as orc

from helpers import NP_DT, TORCH_DT, check_lse, check_out, decode, say, to_dev, to_host

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
_cache = {}


def inputs(key, B=None):
    w = synth.WORKLOADS[key]
    if B is not None:
        w = w.with_batch(B)
    k = (key, w.B)
    if k not in _cache:
        _cache[k] = (w, synth.rank_inputs(w))
    return _cache[k]


def host_send(w, inp):
    """Oracle pack of every rank into a stacked interleaved send buffer (host)."""
    lpd = 4 // w.esize
    send = np.zeros((w.N, w.N, w.B, w.Hpr, w.D + lpd), NP_DT[w.dtype])
    pay, words = orc.interleaved_views_np(send, w.D, w.dtype)
    for r in range(w.N):
        orc.pack(inp["out"][r], inp["lse"][r], pay[r], words[r], w.N)
    return send, pay, words


def check_destinations(w, pay, words, got_out, got_g):
    for p in range(w.N):
        ref, g, mag, _ = orc.combine(pay[:, p], words[:, p], w.dtype, w.base2)
        check_out(decode(to_host(got_out[p], w.dtype), w.dtype), ref, mag, w.dtype, "dest %d" % p)
        if got_g is not None:
            check_lse(got_g[p].cpu().numpy(), g)


INTERLEAVED = [("tiny", None), ("dsv3", None), ("dsv3fp8", None)] + [("longctx", b) for b in synth.LONGCTX_BATCHES]


@pytest.mark.parametrize("key,B", INTERLEAVED)
def test_combine_interleaved_workloads(key, B):
    w, inp = inputs(key, B)
    say("combine interleaved", w.describe())
    send, pay, words = host_send(w, inp)
    dsend = to_dev(send, w.dtype, DEV)
    dpay, dwords = ops.interleaved_views(dsend, w.D)
    out, g = ops.dcp_lse_combine(dpay.transpose(0, 1), dwords.transpose(0, 1), is_lse_base_on_e=not w.base2)
    check_destinations(w, pay, words, out, g)


def test_combine_split_workload():
    """Split peer-inside workload: the combine reads the FlashInfer-shaped
    receive buffers through permuted, non-contiguous views."""
    w, inp = inputs("split")
    say("combine split", w.describe())
    N, B, Hpr, D = w.N, w.B, w.Hpr, w.D
    part = np.zeros((N, B, Hpr, N, D), np.float16)
    stats = np.frombuffer(np.random.default_rng(3).bytes(N * B * Hpr * N * 8), np.float32).reshape(N, B, Hpr, N, 2).copy()
    for r in range(N):
        orc.pack(inp["out"][r], inp["lse"][r], part[r].transpose(2, 0, 1, 3), stats[r][..., 0].transpose(2, 0, 1), N)
    o_out = np.ascontiguousarray(part.transpose(3, 1, 2, 0, 4))       # exchange: [dst, b, hl, src, D]
    s_out = np.ascontiguousarray(stats.transpose(3, 1, 2, 0, 4))
    do = torch.from_numpy(o_out).to(DEV)
    ds = torch.from_numpy(s_out).to(DEV)
    out, g = ops.dcp_lse_combine(do.permute(0, 3, 1, 2, 4), ds[..., 0].permute(0, 3, 1, 2), is_lse_base_on_e=True)
    for p in range(N):
        ref, gr, mag, _ = orc.combine(o_out[p].transpose(2, 0, 1, 3), s_out[p][..., 0].transpose(2, 0, 1), "f16", False)
        check_out(out[p].cpu().numpy(), ref, mag, "f16", "dest %d" % p)
        check_lse(g[p].cpu().numpy(), gr)


@pytest.mark.parametrize("key,B", [("tiny", None), ("dsv3", None), ("longctx", 64), ("split", None), ("dsv3fp8", None)])
def test_end_to_end_pack_exchange_combine(key, B):
    w, inp = inputs(key, B)
    say("end to end", w.describe())
    o = to_dev(inp["out"], w.dtype, DEV)
    l = torch.from_numpy(inp["lse"]).to(DEV)
    if w.layout == "split":
        st = sim.StackedSplit(w.N, w.B, w.H, w.D, TORCH_DT[w.dtype], DEV)
        st.pack(o, l)
        st.exchange()
    else:
        st = sim.StackedInterleaved(w.N, w.B, w.H, w.D, TORCH_DT[w.dtype], DEV)
        st.pack(o, l)
    out, g = st.combine(is_lse_base_on_e=not w.base2)
    # oracle: pack -> exchange -> combine on the host, from the same generated inputs
    _, pay, words = host_send(w, inp)
    check_destinations(w, pay, words, out, g)


# --------------------------------------------------------------------------
# special values, general N, odd shapes, strides, determinism
# --------------------------------------------------------------------------
SPECIALS = [math.nan, math.inf, -math.inf, -2.5, 0.0, 7.25]


@pytest.mark.parametrize("dt", ["f32", "bf16", "f16", "fp8"])
@pytest.mark.parametrize("base2", [False, True])
def test_special_values_every_combination(dt, base2):
    """Every combination of special LSE values over N=3 peers, with NaN and
    +-inf planted in the partials as well."""
    say("specials", dt, base2)
    rows = list(itertools.product(SPECIALS, repeat=3))
    N, B, Hpr, D = 3, len(rows), 1, 64
    lse = np.array(rows, np.float32).T.reshape(N, B, Hpr).copy()
    g = torch.Generator().manual_seed(5)
    o = synth.to_storage(torch.randn(N, B, Hpr, D, generator=g), dt)
    special_o = synth.to_storage(torch.tensor([math.nan, math.inf, -math.inf]), dt)
    rng = np.random.default_rng(2)
    for k in range(60):
        o[rng.integers(N), rng.integers(B), 0, rng.integers(D)] = special_o[k % 3]
    out, gg = ops.dcp_lse_combine(to_dev(o, dt, DEV), torch.from_numpy(lse).to(DEV), is_lse_base_on_e=not base2)
    ref, gr, mag, _ = orc.combine(o, lse, dt, base2)
    check_out(decode(to_host(out, dt), dt), ref, mag, dt)
    check_lse(gg.cpu().numpy(), gr)


@pytest.mark.parametrize("dt", ["f32", "bf16", "f16", "fp8"])
@pytest.mark.parametrize("N", [1, 2, 3, 5, 8, 16, 17, 33])
@pytest.mark.parametrize("D", [64, 100, 512])
def test_general_shapes(dt, N, D):
    """Any N (fixed-N DPP path for 2/4/8/16, looped path otherwise, N = 1
    shortcut), rows that are not 16-byte multiples (D = 100 at 16 bits gives
    200-byte rows: element-granular path), ragged batch and head counts."""
    say("general", dt, N, D)
    B, Hpr, R = 7, 3, 2
    g = torch.Generator().manual_seed(N * 1000 + D)
    o = synth.to_storage(torch.randn(R, N, B, Hpr, D, generator=g), dt)
    rng = np.random.default_rng(N + D)
    lse = rng.normal(0, 4, size=(R, N, B, Hpr)).astype(np.float32)
    lse[0, 0, 1, :] = -np.inf                    # a neutral peer
    lse[1, :, 2, 1] = -np.inf                    # an all-neutral row
    base2 = (N + D) % 2 == 1
    out, gg = ops.dcp_lse_combine(to_dev(o, dt, DEV), torch.from_numpy(lse).to(DEV), is_lse_base_on_e=not base2)
    for r in range(R):
        ref, gr, mag, _ = orc.combine(o[r], lse[r], dt, base2)
        got = decode(to_host(out[r], dt), dt)
        if N == 1:
            assert np.array_equal(to_host(out[r], dt).view(np.uint8), np.ascontiguousarray(o[r, 0]).view(np.uint8))
            assert np.array_equal(gg[r].cpu().numpy().view(np.uint32), lse[r, 0].view(np.uint32))
        else:
            check_out(got, ref, mag, dt, "r=%d" % r)
            check_lse(gg[r].cpu().numpy(), gr)


@pytest.mark.parametrize("dt,N,D", [("bf16", 8, 400), ("f16", 16, 384), ("f32", 4, 1000), ("bf16", 2, 512),
                                    ("fp8", 8, 1024), ("fp8", 16, 800)])
@pytest.mark.parametrize("B", [5, 40, 300])
def test_row_per_wave_kernel_guards_and_ragged_rows(dt, N, D, B):
    """Rows of 768 bytes and more take the row-per-wave kernel: at B = 5 (40
    to 80 row segments) in the latency order (payload loads issued before
    the LSE reduction) in 4-byte vectors, at B = 40 (320 to 640) in the same
    order in 16-byte vectors, at B = 300 (2400 or more) in the bandwidth
    order.  Rows that are not a multiple of 64 vectors leave idle lanes in
    their last segment;
    NaN and +-inf planted in the payload force the guarded re-read; special
    LSE values and an all-neutral row are mixed in."""
    say("row-per-wave", dt, N, D, B)
    Hpr = 8
    g = torch.Generator().manual_seed(N * 7 + D + B)
    o = synth.to_storage(torch.randn(N, B, Hpr, D, generator=g), dt)
    rng = np.random.default_rng(N + D + B)
    lse = rng.normal(0, 4, size=(N, B, Hpr)).astype(np.float32)
    for k in range(40):
        lse[rng.integers(N), rng.integers(B), rng.integers(Hpr)] = [np.nan, np.inf, -np.inf][k % 3]
    lse[:, 0, 0] = -np.inf
    special_o = synth.to_storage(torch.tensor([math.nan, math.inf, -math.inf]), dt)
    for k in range(100):
        o[rng.integers(N), rng.integers(B), rng.integers(Hpr), rng.integers(D)] = special_o[k % 3]
    base2 = B % 2 == 0
    out, gg = ops.dcp_lse_combine(to_dev(o, dt, DEV), torch.from_numpy(lse).to(DEV), is_lse_base_on_e=not base2)
    ref, gr, mag, _ = orc.combine(o, lse, dt, base2)
    check_out(decode(to_host(out, dt), dt), ref, mag, dt)
    check_lse(gg.cpu().numpy(), gr)


@pytest.mark.parametrize("dt,N,D,B,Hpr", [
    ("bf16", 8, 512, 4096, 8),     # 32768 rows, 32 MiB of output: payload loads first, plain stores
    ("bf16", 8, 512, 8192, 8),     # 65536 rows, 64 MiB: payload loads first, nontemporal stores
    ("f32", 2, 1000, 1100, 8),     # 35200 row segments (4 per row), 34 MiB
    ("fp8", 4, 1024, 8192, 8),     # 65536 rows of 1 KB fp8, 64 MiB
    ("bf16", 16, 512, 10923, 3),   # 32769 rows: the last 2-wave workgroup's second wave is past the end
])
def test_row_per_wave_kernel_guards_large_launches(dt, N, D, B, Hpr):
    """Launches of 32768 row segments and more issue the payload loads before
    the LSE reduction, and merged outputs of 64 MiB and more go out with
    nontemporal stores: NaN and +-inf planted in the payload force the
    guarded re-read there too, with special LSE values and all-neutral rows;
    every output element and every G is compared.  A wave past the last row
    segment redoes the first one and must store nothing: out and G are
    written into buffers with random guard bands around them, which must
    come back unchanged."""
    say("row-per-wave large launch", dt, N, D, B, Hpr)
    g = torch.Generator().manual_seed(N * 7 + D + B)
    o = synth.to_storage(torch.randn(N, B, Hpr, D, generator=g), dt)
    rng = np.random.default_rng(N + D + B)
    lse = rng.normal(0, 4, size=(N, B, Hpr)).astype(np.float32)
    for k in range(300):
        lse[rng.integers(N), rng.integers(B), rng.integers(Hpr)] = [np.nan, np.inf, -np.inf][k % 3]
    lse[:, 0, 0] = -np.inf
    lse[:, B - 1, Hpr - 1] = -np.inf
    special_o = synth.to_storage(torch.tensor([math.nan, math.inf, -math.inf]), dt)
    for k in range(600):
        o[rng.integers(N), rng.integers(B), rng.integers(Hpr), rng.integers(D)] = special_o[k % 3]
    # out and G inside guarded byte buffers
    esz = np.dtype(NP_DT[dt]).itemsize
    nout, nlse, guard = B * Hpr * D * esz, B * Hpr * 4, 4096
    rng_g = np.random.default_rng(B + Hpr)
    hout = np.frombuffer(rng_g.bytes(nout + 2 * guard), np.uint8).copy()
    hlse = np.frombuffer(rng_g.bytes(nlse + 2 * guard), np.uint8).copy()
    bout, blse = torch.from_numpy(hout).to(DEV), torch.from_numpy(hlse).to(DEV)
    out_v = bout[guard:guard + nout].view(TORCH_DT[dt]).view(B, Hpr, D)
    lse_v = blse[guard:guard + nlse].view(torch.float32).view(B, Hpr)
    out, gg = ops.dcp_lse_combine(to_dev(o, dt, DEV), torch.from_numpy(lse).to(DEV), is_lse_base_on_e=False,
                                  out=out_v, out_lse=lse_v)
    ref, gr, mag, _ = orc.combine(o, lse, dt, True)
    check_out(decode(to_host(out, dt), dt), ref, mag, dt)
    check_lse(gg.cpu().numpy(), gr)
    gout, glse = bout.cpu().numpy(), blse.cpu().numpy()
    for got, host, n in ((gout, hout, nout), (glse, hlse, nlse)):
        assert np.array_equal(got[:guard], host[:guard]) and np.array_equal(got[guard + n:], host[guard + n:]), \
            "a store landed outside the output"


@pytest.mark.parametrize("dt,N,B,Hpr,D", [
    ("bf16", 8, 5, 4, 512),      # row-per-wave kernel, latency order
    ("bf16", 8, 160, 16, 512),   # row-per-wave kernel, bandwidth order (2560 rows)
    ("f32", 4, 6, 3, 1000),      # several segments per row
    ("f16", 4, 9, 5, 128),       # short-row kernel
    ("f32", 17, 4, 3, 64),       # any-N path
    ("bf16", 3, 4, 2, 100),      # element-granular rows
    ("f32", 1, 4, 3, 64),        # N = 1 copy onto itself
    ("fp8", 8, 5, 4, 1024),      # fp8, row-per-wave kernel
    ("fp8", 4, 9, 5, 128),       # fp8, short-row kernel
])
def test_out_may_alias_peer_zero(dt, N, B, Hpr, D):
    """out may be exactly recv_o's peer 0 rows: the merge lands in place in
    the first received partial, and matches the oracle on the original input."""
    say("alias", dt, N, B, Hpr, D)
    g = torch.Generator().manual_seed(N * 31 + D)
    o = synth.to_storage(torch.randn(N, B, Hpr, D, generator=g), dt)
    lse = np.random.default_rng(D + N).normal(0, 3, size=(N, B, Hpr)).astype(np.float32)
    lse[:, 0, 0] = -np.inf
    d_o = to_dev(o, dt, DEV)
    d_l = torch.from_numpy(lse).to(DEV)
    out, gg = ops.dcp_lse_combine(d_o, d_l, is_lse_base_on_e=True, out=d_o[0])
    assert out.data_ptr() == d_o.data_ptr()
    got = to_host(d_o[0], dt)
    if N == 1:
        assert np.array_equal(got.view(np.uint8), o[0].view(np.uint8))
        return
    ref, gr, mag, _ = orc.combine(o, lse, dt, False)
    check_out(decode(got, dt), ref, mag, dt)
    check_lse(gg.cpu().numpy(), gr)
    # the other peers' rows are untouched
    assert np.array_equal(to_host(d_o[1:], dt).view(np.uint8), o[1:].view(np.uint8))


def test_single_rank_identity_keeps_nan_and_inf_bits():
    o = np.random.default_rng(0).normal(size=(1, 3, 2, 64)).astype(np.float32)
    o[0, 0, 0, :3] = [np.nan, np.inf, -np.inf]
    lse = np.array([[[np.nan, 1.0], [np.inf, -np.inf], [2.0, 3.0]]], np.float32)
    out, g = ops.dcp_lse_combine(torch.from_numpy(o).to(DEV), torch.from_numpy(lse).to(DEV))
    assert np.array_equal(out.cpu().numpy().view(np.uint32), o[0].view(np.uint32))
    assert np.array_equal(g.cpu().numpy().view(np.uint32), lse[0].view(np.uint32))


def test_large_lse_magnitudes_and_spread():
    """LSEs near 1e4 (G's fp32 rounding dominates) and spreads of hundreds
    (weights underflow to zero) stay within tolerance."""
    rng = np.random.default_rng(4)
    N, B, Hpr, D = 8, 16, 4, 128
    o = rng.normal(size=(N, B, Hpr, D)).astype(np.float32)
    lse = (rng.normal(0, 200, size=(N, B, Hpr)) + 1e4).astype(np.float32)
    for base2 in (False, True):
        out, g = ops.dcp_lse_combine(torch.from_numpy(o).to(DEV), torch.from_numpy(lse).to(DEV),
                                     is_lse_base_on_e=not base2)
        ref, gr, mag, _ = orc.combine(o, lse, "f32", base2)
        check_out(out.cpu().numpy(), ref, mag, "f32")
        check_lse(g.cpu().numpy(), gr)


def test_no_lse_output_and_preallocated_out():
    w, inp = inputs("tiny")
    send, pay, words = host_send(w, inp)
    dsend = to_dev(send, w.dtype, DEV)
    dpay, dwords = ops.interleaved_views(dsend, w.D)
    pre = torch.full((w.N, w.B, w.Hpr, w.D), 123.0, device=DEV)
    out, g = ops.dcp_lse_combine(dpay.transpose(0, 1), dwords.transpose(0, 1), is_lse_base_on_e=True,
                                 return_lse=False, out=pre)
    assert g is None and out.data_ptr() == pre.data_ptr()
    check_destinations(w, pay, words, out, None)


def test_combine_deterministic():
    w, inp = inputs("longctx", 64)
    send, _, _ = host_send(w, inp)
    dsend = to_dev(send, w.dtype, DEV)
    dpay, dwords = ops.interleaved_views(dsend, w.D)
    a = ops.dcp_lse_combine(dpay.transpose(0, 1), dwords.transpose(0, 1), is_lse_base_on_e=False)
    b = ops.dcp_lse_combine(dpay.transpose(0, 1), dwords.transpose(0, 1), is_lse_base_on_e=False)
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
    assert torch.equal(a[1].view(torch.int32), b[1].view(torch.int32))


def test_neutral_rank_changes_nothing_on_gpu():
    """Appending a (0, -inf) peer leaves the GPU result within tolerance of the
    oracle without it (the oracle's own result is exactly unchanged)."""
    rng = np.random.default_rng(8)
    N, B, Hpr, D = 4, 9, 5, 256
    o = synth.to_storage(torch.randn(N + 1, B, Hpr, D, generator=torch.Generator().manual_seed(1)), "bf16")
    o[N] = 0
    lse = rng.normal(0, 3, size=(N + 1, B, Hpr)).astype(np.float32)
    lse[N] = -np.inf
    out, g = ops.dcp_lse_combine(to_dev(o, "bf16", DEV), torch.from_numpy(lse).to(DEV), is_lse_base_on_e=True)
    ref, gr, mag, _ = orc.combine(o[:N], lse[:N], "bf16", False)
    check_out(decode(to_host(out, "bf16"), "bf16"), ref, mag, "bf16")
    check_lse(g.cpu().numpy(), gr)
