"""GPU parity of dcp_lse_combine_inplace against the fp64 oracle, including
the full-size in-place workload (8 ranks x [16384, 96, 512] fp32 = 24 GiB)
and its reduce-scatter flavour, both checked on every row."""
import numpy as np
import pytest
import torch

from lse_weighted_merge_dcp_amd import ops, sim, synth
from oracle import oracle as orc

from helpers import check_lse, check_out, check_scaled, decode, say, to_dev, to_host

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def kimi_small(T):
    w = synth.WORKLOADS["kimi"].with_batch(T)
    return w, synth.rank_inputs(w)


@pytest.mark.parametrize("T", [48, 5])
def test_inplace_kimi_shape_small_T(T):
    """The in-place workload's shape and LSE law at a small token count:
    N=8 ranks, H=96, D=512 fp32, base e, 0.1% NaN/+inf/-inf LSE entries."""
    w, inp = kimi_small(T)
    say("inplace kimi T=%d" % T)
    lse = inp["lse"].copy()
    if T == 5:                       # plant every special value at least once
        lse[0, 0, 0] = np.nan; lse[3, 1, 2] = np.inf; lse[:, 2, 3] = -np.inf; lse[5, 4, 95] = -np.inf
    part = torch.from_numpy(inp["out"]).to(DEV)
    l = torch.from_numpy(lse).to(DEV)
    H = w.H
    for r in (0, 3, 7):   # each simulated rank's head slice, then the full merge
        h0, h1 = 12 * r, 12 * r + 12
        p = part.clone()
        out, g = ops.cp_lse_combine_inplace(p, l, h0=h0, h1=h1, return_lse=True)
        scaled, ref, gr, mag = orc.inplace(inp["out"], lse, "f32", False, h0=h0, h1=h1)
        check_out(out.cpu().numpy(), ref, mag, "f32", "slice %d" % r)
        check_lse(g.cpu().numpy(), gr)
        check_scaled(p.cpu().numpy(), scaled, "f32")
    out = ops.cp_lse_combine_inplace(part, l, h0=0, h1=H)
    scaled, ref, gr, mag = orc.inplace(inp["out"], lse, "f32", False)
    check_out(out.cpu().numpy(), ref, mag, "f32", "full")
    check_scaled(part.cpu().numpy(), scaled, "f32")


@pytest.mark.parametrize("dt", ["f32", "bf16", "f16", "fp8"])
@pytest.mark.parametrize("N,P,rank0", [(8, 8, 0), (4, 1, 2), (8, 3, 5), (3, 3, 0), (17, 17, 0), (17, 2, 7), (2, 2, 0), (16, 16, 0)])
def test_inplace_held_subsets_and_dtypes(dt, N, P, rank0):
    """P of the N ranks' partials held (rank0 .. rank0+P-1): the single-rank
    case P = 1 is what one GPU of a real group runs before its all-reduce."""
    say("inplace subset", dt, N, P, rank0)
    T, H, D = 6, 10, 192
    g = torch.Generator().manual_seed(N * 31 + P)
    part = synth.to_storage(torch.randn(P, T, H, D, generator=g), dt)
    part[0, 1, 2, 5] = synth.to_storage(torch.tensor([float("nan")]), dt)[0]
    lse = np.random.default_rng(N).normal(1, 3, size=(N, T, H)).astype(np.float32)
    lse[rank0, 2, 4] = np.nan
    lse[:, 3, 5] = -np.inf
    base2 = (N + P) % 2 == 0
    h0, h1 = 3, 8
    p = to_dev(part, dt, DEV)
    out, gg = ops.cp_lse_combine_inplace(p, torch.from_numpy(lse).to(DEV), h0=h0, h1=h1, rank0=rank0,
                                         is_lse_base_on_e=not base2, return_lse=True)
    scaled, ref, gr, mag = orc.inplace(part, lse, dt, base2, rank0=rank0, h0=h0, h1=h1)
    check_out(decode(to_host(out, dt), dt), ref, mag, dt)
    check_lse(gg.cpu().numpy(), gr)
    check_scaled(decode(to_host(p, dt), dt), scaled, dt)


@pytest.mark.parametrize("dt,D", [("f32", 512), ("f32", 520), ("f32", 192), ("bf16", 100), ("f16", 512),
                                  ("bf16", 1000), ("fp8", 2048), ("fp8", 100)])
@pytest.mark.parametrize("want_out", [True, False])
def test_inplace_single_rank_segment_groups(dt, D, want_out):
    """P = 1, one rank scaling its own partial: each row group takes two
    segments of a row.  Rows of an odd number of segments, a partly filled
    second segment, rows that are not 16-byte multiples (element-wise path),
    with and without the output slice."""
    say("inplace single rank", dt, D, want_out)
    N, T, H, rank0 = 8, 5, 12, 3
    g = torch.Generator().manual_seed(D)
    part = synth.to_storage(torch.randn(1, T, H, D, generator=g), dt)
    part[0, 2, 7, D - 1] = synth.to_storage(torch.tensor([float("inf")]), dt)[0]
    lse = np.random.default_rng(D).normal(0, 3, size=(N, T, H)).astype(np.float32)
    lse[rank0, 1, 3] = np.nan
    lse[:, 4, 0] = -np.inf
    lse[5, 0, 9] = np.inf
    p = to_dev(part, dt, DEV)
    h0, h1 = 2, 11
    res = ops.cp_lse_combine_inplace(p, torch.from_numpy(lse).to(DEV), h0=h0, h1=h1, rank0=rank0,
                                     return_lse=want_out, want_out=want_out)
    scaled, ref, gr, mag = orc.inplace(part, lse, dt, False, rank0=rank0, h0=h0, h1=h1)
    check_scaled(decode(to_host(p, dt), dt), scaled, dt)
    if want_out:
        out, gg = res
        check_out(decode(to_host(out, dt), dt), ref, mag, dt)
        check_lse(gg.cpu().numpy(), gr)


def test_inplace_scale_only_and_single_rank():
    rng = np.random.default_rng(3)
    part = rng.normal(size=(4, 3, 6, 64)).astype(np.float32)
    lse = rng.normal(size=(4, 3, 6)).astype(np.float32)
    p = torch.from_numpy(part).to(DEV)
    r = ops.cp_lse_combine_inplace(p, torch.from_numpy(lse).to(DEV), want_out=False)
    assert r is None
    scaled, _, _, _ = orc.inplace(part, lse, "f32", False)
    check_scaled(p.cpu().numpy(), scaled, "f32")
    # N == 1: the partial is left as it is and the slice is a bit copy
    one = part[:1].copy()
    one[0, 0, 0, 0] = np.nan
    p1 = torch.from_numpy(one).to(DEV)
    out, g = ops.cp_lse_combine_inplace(p1, torch.from_numpy(lse[:1]).to(DEV), h0=1, h1=4, return_lse=True)
    assert np.array_equal(p1.cpu().numpy().view(np.uint32), one.view(np.uint32))
    assert np.array_equal(out.cpu().numpy().view(np.uint32), one[0][:, 1:4].view(np.uint32))
    assert np.array_equal(g.cpu().numpy().view(np.uint32), lse[0][:, 1:4].view(np.uint32))


def test_reduce_scatter_flavour_through_strided_combine():
    """The merged head slice without the write-back: dcp_unpack_combine over a
    strided view of the partial stack (heads [h0,h1)) equals the in-place
    merge's slice."""
    w, inp = kimi_small(16)
    lse = torch.from_numpy(inp["lse"]).to(DEV)
    part = torch.from_numpy(inp["out"]).to(DEV)
    h0, h1 = 24, 36
    rs, g = ops.dcp_lse_combine(part[:, :, h0:h1], lse[:, :, h0:h1], is_lse_base_on_e=True)
    scaled, ref, gr, mag = orc.inplace(inp["out"], inp["lse"], "f32", False, h0=h0, h1=h1)
    check_out(rs.cpu().numpy(), ref, mag, "f32")
    check_lse(g.cpu().numpy(), gr)
    # all 8 ranks' slices in one launch (the benchmarked form), with every
    # special LSE value planted
    lse_np = inp["lse"].copy()
    lse_np[0, 0, 0] = np.nan; lse_np[3, 1, 13] = np.inf; lse_np[:, 2, 30] = -np.inf; lse_np[5, 4, 95] = -np.inf
    out, g = sim.reduce_scatter_merge(part, torch.from_numpy(lse_np).to(DEV))
    _, ref, gr, mag = orc.inplace(inp["out"], lse_np, "f32", False)
    check_out(out.cpu().numpy(), ref, mag, "f32")
    check_lse(g.cpu().numpy(), gr)


# ---------------------------------------------------------------------------
# Full size, every row: 8 x [16384, 96, 512] fp32 partials (24 GiB) merged in
# the launch configurations the benchmark times -- first the reduce-scatter
# flavour (every rank's head slice in one launch; the partials stay as they
# are), then in place.  Each test below takes one block of 2048 tokens: it
# draws that block's pristine partials again from their seeds, runs the
# oracle on them in pieces of 256 tokens, and compares every scaled partial
# of all 8 ranks, every merged row and every G of both calls.
# ---------------------------------------------------------------------------
FULL_PIECE = 256


@pytest.fixture(scope="module")
def full_kimi():
    w = synth.WORKLOADS["kimi"]
    say("inplace full size", w.describe())
    part = synth.kimi_partial_device(w, DEV)
    lse_np = synth.kimi_lse(w)
    lse = torch.from_numpy(lse_np).to(DEV)
    rs_out, rs_g = sim.reduce_scatter_merge(part, lse)
    torch.cuda.synchronize()
    # the reduce-scatter flavour writes no partial: every byte is still the
    # seeded draw (this also proves the block-wise redraw below exact)
    for t0 in range(0, w.B, synth.KIMI_TOKEN_BLOCK):
        blk = synth.kimi_partial_block_device(w, DEV, t0)
        assert torch.equal(part[:, t0:t0 + blk.shape[1]].view(torch.int32), blk.view(torch.int32)), t0
        del blk
    out, g = ops.cp_lse_combine_inplace(part, lse, return_lse=True)
    torch.cuda.synchronize()
    say("inplace full size: both calls done")
    yield w, part, lse_np, out, g, rs_out, rs_g
    del part, out, g, rs_out, rs_g
    torch.cuda.empty_cache()


@pytest.mark.parametrize("t0", list(range(0, synth.WORKLOADS["kimi"].B, synth.KIMI_TOKEN_BLOCK)))
def test_inplace_full_size_every_row(full_kimi, t0):
    w, part, lse_np, out, g, rs_out, rs_g = full_kimi
    say("inplace full size: tokens", t0, t0 + synth.KIMI_TOKEN_BLOCK)
    pristine = synth.kimi_partial_block_device(w, DEV, t0).cpu().numpy()
    for p0 in range(0, pristine.shape[1], FULL_PIECE):
        a, b = t0 + p0, t0 + p0 + FULL_PIECE
        scaled, ref, gr, mag = orc.inplace(pristine[:, p0:p0 + FULL_PIECE], lse_np[:, a:b], "f32", False)
        where = "tokens [%d, %d)" % (a, b)
        check_scaled(part[:, a:b], scaled, "f32", "scaled partials, " + where)
        check_out(out[a:b], ref, mag, "f32", "in-place merge, " + where)
        check_lse(g[a:b].cpu().numpy(), gr)
        check_out(rs_out[a:b], ref, mag, "f32", "reduce-scatter merge, " + where)
        check_lse(rs_g[a:b].cpu().numpy(), gr)
