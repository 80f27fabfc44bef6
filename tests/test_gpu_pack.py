"""GPU parity of dcp_pack: bit-exact against the oracle, byte for byte over the
whole destination allocation.

Each destination lives inside a larger byte buffer pre-filled with random
bytes (guard bands before and after, and every byte the map does not
address, e.g. stats slot 1): after the pack, every byte must equal what the
oracle's pack leaves in a host copy of the same pre-filled buffer.
"""
import numpy as np
import pytest
import torch

from lse_weighted_merge_dcp_amd import ops, synth
from oracle import oracle as orc

from helpers import NP_DT, TORCH_DT, say, to_dev

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
GUARD = 4096
_cache = {}


def inputs(key, B=None):
    w = synth.WORKLOADS[key]
    if B is not None:
        w = w.with_batch(B)
    k = (key, w.B)
    if k not in _cache:
        _cache[k] = (w, synth.rank_inputs(w))
    return _cache[k]


def guarded(nbytes, seed):
    """(device buffer, host copy): random bytes with GUARD bytes on each side."""
    host = np.frombuffer(np.random.default_rng(seed).bytes(nbytes + 2 * GUARD), np.uint8).copy()
    return torch.from_numpy(host).to(DEV), host


def dev_view(buf, dtype, shape):
    n = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
    return buf[GUARD:GUARD + n].view(dtype).view(shape)


def host_view(host, npdt, shape):
    n = int(np.prod(shape)) * np.dtype(npdt).itemsize
    return host[GUARD:GUARD + n].view(npdt).reshape(shape)


INTERLEAVED = [("tiny", None), ("dsv3", None), ("dsv3fp8", None)] + [("longctx", b) for b in synth.LONGCTX_BATCHES]


@pytest.mark.parametrize("key,B", INTERLEAVED)
def test_pack_interleaved_workloads(key, B):
    """All N ranks pack their peer-outer interleaved send buffers [N,B,Hpr,D+lpd]
    (stacked as send[src, peer, ...]) in one launch."""
    w, inp = inputs(key, B)
    say("pack interleaved", w.describe())
    N, Bt, H, D, dt = w.N, w.B, w.H, w.D, w.dtype
    lpd = 4 // w.esize
    shape = (N, N, Bt, w.Hpr, D + lpd)
    nbytes = int(np.prod(shape)) * w.esize
    buf, host = guarded(nbytes, seed=w.index * 100 + Bt)
    send = dev_view(buf, TORCH_DT[dt], shape)
    pay, words = ops.interleaved_views(send, D)
    ops.dcp_pack_a2a_send(to_dev(inp["out"], dt, DEV), torch.from_numpy(inp["lse"]).to(DEV), pay, words)
    got = buf.cpu().numpy()
    hsend = host_view(host, NP_DT[dt], shape)
    hpay, hwords = orc.interleaved_views_np(hsend, D, dt)
    for r in range(N):
        orc.pack(inp["out"][r], inp["lse"][r], hpay[r], hwords[r], N)
    assert np.array_equal(got, host), "pack differs at %d bytes" % int((got != host).sum())


def test_pack_large_send_blocks_fp8_two_lse_words():
    """A pack whose send blocks span 768 MiB or more writes them with the
    nontemporal hint; fp8 rows of 516 bytes (two LSE words in most
    wave-steps) at 811 MB, compared byte for byte with guard bands."""
    N, B, H, D, dt = 16, 768, 128, 512, "fp8"
    Hpr = H // N
    say("pack large fp8", N, B, H, D)
    g = torch.Generator().manual_seed(5)
    out = synth.to_storage(torch.randn(N, B, H, D, generator=g), dt)
    lse = np.random.default_rng(5).normal(10, 3, size=(N, B, H)).astype(np.float32)
    shape = (N, N, B, Hpr, D + 4)
    nbytes = int(np.prod(shape))
    assert nbytes >= 768 << 20
    buf, host = guarded(nbytes, seed=17)
    send = dev_view(buf, TORCH_DT[dt], shape)
    pay, words = ops.interleaved_views(send, D)
    ops.dcp_pack_a2a_send(to_dev(out, dt, DEV), torch.from_numpy(lse).to(DEV), pay, words)
    got = buf.cpu().numpy()
    hsend = host_view(host, NP_DT[dt], shape)
    hpay, hwords = orc.interleaved_views_np(hsend, D, dt)
    for r in range(N):
        orc.pack(out[r], lse[r], hpay[r], hwords[r], N)
    assert np.array_equal(got, host), "pack differs at %d bytes" % int((got != host).sum())
    del buf, send, pay, words
    torch.cuda.empty_cache()


STREAM_SHAPES = [
    ("bf16", 8, 5, 16, 512),    # the decode shape, ragged batch
    ("bf16", 4, 3, 4, 512),     # small peer blocks (Hpr * W = 4112 B)
    ("f32", 2, 6, 8, 256),      # fp32 rows of 1 KB (W = 1028)
    ("f32", 4, 2, 12, 512),     # 2 KB rows: several LSE-free wave-steps per row
    ("f16", 2, 3, 8, 1024),     # 2 KB fp16 rows
    ("bf16", 1, 4, 8, 768),     # a single peer (N = 1)
    ("bf16", 2, 3, 3, 512),     # Hpr * W not a multiple of 16: falls back to the row kernel
    ("bf16", 2, 3, 8, 504),     # rows just under 1 KB (W = 1012): two LSE words in some wave-steps
    ("bf16", 4, 3, 8, 256),     # W = 516: two LSE words in most wave-steps
    ("f32", 2, 5, 8, 127),      # W = 512 (128 dwords, the smallest stream row)
    ("bf16", 2, 3, 4, 382),     # W = 768
    ("bf16", 2, 3, 8, 200),     # rows under 512 B (W = 404): row kernel
    ("fp8", 8, 5, 16, 512),     # the fp8 decode shape (W = 516, lpd = 4)
    ("fp8", 8, 5, 16, 1024),    # fp8 rows of 1 KB (W = 1028)
    ("fp8", 4, 3, 8, 2044),     # fp8 rows of 2 KB
]


@pytest.mark.parametrize("dt,N,B,Hpr,D", STREAM_SHAPES)
def test_pack_interleaved_stream_shapes(dt, N, B, Hpr, D):
    """Interleaved send buffers of several shapes, two simulated source ranks
    (R = 2), checked byte for byte with guard bands."""
    say("pack stream shapes", dt, N, B, Hpr, D)
    R, H = 2, N * Hpr
    esz = np.dtype(NP_DT[dt]).itemsize
    lpd = 4 // esz
    g = torch.Generator().manual_seed(N * 31 + D)
    out = synth.to_storage(torch.randn(R, B, H, D, generator=g), dt)
    lse = np.random.default_rng(D + B).normal(size=(R, B, H)).astype(np.float32)
    lse[0, 0, :2] = [np.nan, -np.inf]
    shape = (R, N, B, Hpr, D + lpd)
    buf, host = guarded(int(np.prod(shape)) * esz, seed=D + N)
    send = dev_view(buf, TORCH_DT[dt], shape)
    pay, words = ops.interleaved_views(send, D)
    ops.dcp_pack_a2a_send(to_dev(out, dt, DEV), torch.from_numpy(lse).to(DEV), pay, words)
    hsend = host_view(host, NP_DT[dt], shape)
    hpay, hwords = orc.interleaved_views_np(hsend, D, dt)
    for r in range(R):
        orc.pack(out[r], lse[r], hpay[r], hwords[r], N)
    got = buf.cpu().numpy()
    assert np.array_equal(got, host), "pack differs at %d bytes" % int((got != host).sum())


# Calls of 131,072 wave-steps and more run in 4-wave workgroups whose XCDs
# take turns on chunks of 128; the long-context workloads above reach them
# with nontemporal loads (and stores at B = 512).  These cases reach the same
# launch with ragged batches, plain loads and rows of 516 bytes, and the
# 8-wave launch below it (32,768 to 131,071 wave-steps, the LSE words through
# scalar loads) with nontemporal loads.
LARGE_SHAPES = [
    ("bf16", 16, 16, 60, 8, 512),   # nontemporal source loads, B = 4 * 15
    ("bf16", 16, 16, 58, 8, 512),   # B = 2 * 29
    ("bf16", 16, 16, 57, 8, 512),   # B odd
    ("bf16", 16, 64, 64, 1, 518),   # Hpr = 1, blocks of 65 chunks, 65 MiB of source: plain loads
    ("f32", 16, 16, 112, 8, 128),   # rows of 516 B: two LSE words in most wave-steps
    ("bf16", 16, 16, 50, 8, 512),   # 115,200 wave-steps, 100 MiB of source: 8-wave launch with nontemporal loads
]


@pytest.mark.parametrize("dt,R,N,B,Hpr,D", LARGE_SHAPES)
def test_pack_large_launch_shapes(dt, R, N, B, Hpr, D):
    """Large interleaved packs of R source ranks, byte for byte with guard
    bands; NaN, -inf and +inf LSEs among them."""
    say("pack large launch shapes", dt, R, N, B, Hpr, D)
    H = N * Hpr
    esz = np.dtype(NP_DT[dt]).itemsize
    lpd = 4 // esz
    g = torch.Generator().manual_seed(B * 7 + D)
    out = synth.to_storage(torch.randn(R, B, H, D, generator=g), dt)
    lse = np.random.default_rng(B + D).normal(5, 4, size=(R, B, H)).astype(np.float32)
    lse[0, 0, :2] = [np.nan, -np.inf]
    lse[R - 1, B - 1, -1] = np.inf
    shape = (R, N, B, Hpr, D + lpd)
    buf, host = guarded(int(np.prod(shape)) * esz, seed=B + N)
    send = dev_view(buf, TORCH_DT[dt], shape)
    pay, words = ops.interleaved_views(send, D)
    ops.dcp_pack_a2a_send(to_dev(out, dt, DEV), torch.from_numpy(lse).to(DEV), pay, words)
    hsend = host_view(host, NP_DT[dt], shape)
    hpay, hwords = orc.interleaved_views_np(hsend, D, dt)
    for r in range(R):
        orc.pack(out[r], lse[r], hpay[r], hwords[r], N)
    got = buf.cpu().numpy()
    assert np.array_equal(got, host), "pack differs at %d bytes" % int((got != host).sum())
    del buf, send, pay, words
    torch.cuda.empty_cache()


SPLIT = [("f16", 4, 256, 16, 128), ("bf16", 2, 4, 8, 128), ("bf16", 4, 1, 16, 512), ("f32", 8, 3, 2, 64),
         ("fp8", 4, 8, 16, 128)]


@pytest.mark.parametrize("dt,N,B,Hpr,D", SPLIT)
def test_pack_split_peer_inside(dt, N, B, Hpr, D):
    """Peer-inside split layout through permuted views: partial_o [B,Hpr,N,D]
    and stats [B,Hpr,N,2] with slot 1 pre-filled and never touched.  The first
    case is the split workload (N=4, B=256, H=64, D=128 fp16); the bf16 cases
    are the shapes of the sglang report's split-layout test."""
    say("pack split", dt, N, B, Hpr, D)
    H = N * Hpr
    rng = np.random.default_rng(N * 1000 + B)
    g = torch.Generator().manual_seed(B * 7 + N)
    o32 = torch.randn(N, B, H, D, generator=g)
    out = synth.to_storage(o32, dt)
    lse = rng.normal(0, 3, size=(N, B, H)).astype(np.float32)
    esz = np.dtype(NP_DT[dt]).itemsize
    pshape, sshape = (N, B, Hpr, N, D), (N, B, Hpr, N, 2)
    pbuf, phost = guarded(int(np.prod(pshape)) * esz, seed=1)
    sbuf, shost = guarded(int(np.prod(sshape)) * 4, seed=2)
    part = dev_view(pbuf, TORCH_DT[dt], pshape)
    stats = dev_view(sbuf, torch.float32, sshape)
    ops.dcp_pack_a2a_send(to_dev(out, dt, DEV), torch.from_numpy(lse).to(DEV),
                          part.permute(0, 3, 1, 2, 4), stats[..., 0].permute(0, 3, 1, 2))
    hp = host_view(phost, NP_DT[dt], pshape)
    hs = host_view(shost, np.float32, sshape)
    for r in range(N):
        orc.pack(out[r], lse[r], hp[r].transpose(2, 0, 1, 3), hs[r][..., 0].transpose(2, 0, 1), N)
    assert np.array_equal(pbuf.cpu().numpy(), phost)
    assert np.array_equal(sbuf.cpu().numpy(), shost)


@pytest.mark.parametrize("dt,N,B,H,D,src_off,dst_off", [
    ("bf16", 2, 5, 6, 7, 1, 1),     # odd element offsets and a 14-byte row: 2-byte accesses
    ("f16", 3, 4, 9, 12, 0, 2),     # 24-byte rows, 4-byte aligned: 8-byte accesses
    ("f32", 4, 3, 8, 5, 1, 3),      # 20-byte rows: 4-byte accesses
    ("bf16", 4, 9, 8, 72, 0, 0),    # 144-byte rows: 16-byte accesses, ragged row groups
    ("f32", 2, 2, 2, 1024, 0, 0),   # 4 KiB rows: several steps per row
    ("fp8", 2, 5, 6, 7, 1, 3),      # fp8: 7-byte rows at odd byte offsets: 1-byte accesses
    ("fp8", 3, 4, 9, 14, 0, 2),     # fp8: 14-byte rows, 2-byte aligned: 2-byte accesses
    ("fp8", 4, 9, 8, 144, 0, 0),    # fp8: 144-byte rows: 16-byte accesses
])
def test_pack_odd_shapes_and_offsets(dt, N, B, H, D, src_off, dst_off):
    say("pack odd", dt, N, B, H, D, src_off, dst_off)
    Hpr = H // N
    lpd = 4 // np.dtype(NP_DT[dt]).itemsize
    g = torch.Generator().manual_seed(D)
    src_full = synth.to_storage(torch.randn(B * H * D + src_off, generator=g), dt)
    src = src_full[src_off:].reshape(B, H, D)
    lse = np.random.default_rng(D).normal(size=(B, H)).astype(np.float32)
    Dp = D + lpd + 1   # padded rows: the destination row stride is not D + lpd
    esz = np.dtype(NP_DT[dt]).itemsize
    nbytes = (N * B * Hpr * Dp + dst_off) * esz
    buf, host = guarded(nbytes, seed=D + 5)
    flat = buf[GUARD:GUARD + nbytes].view(TORCH_DT[dt])
    dst = flat[dst_off:].view(N, B, Hpr, Dp)[..., :D]
    lbuf, lhost = guarded(N * B * Hpr * 4 * 2, seed=D + 6)
    dst_lse = lbuf[GUARD:GUARD + N * B * Hpr * 8].view(torch.float32).view(N, B, Hpr, 2)[..., 1]
    src_dev = to_dev(src_full, dt, DEV)[src_off:].view(B, H, D)
    ops.dcp_pack_a2a_send(src_dev, torch.from_numpy(lse).to(DEV), dst, dst_lse)
    hflat = host[GUARD:GUARD + nbytes].view(NP_DT[dt])
    hdst = hflat[dst_off:dst_off + N * B * Hpr * Dp].reshape(N, B, Hpr, Dp)[..., :D]
    hl = lhost[GUARD:GUARD + N * B * Hpr * 8].view(np.float32).reshape(N, B, Hpr, 2)[..., 1]
    orc.pack(src, lse, hdst, hl, N)
    assert np.array_equal(buf.cpu().numpy(), host)
    assert np.array_equal(lbuf.cpu().numpy(), lhost)


def test_pack_zero_batch_is_noop():
    out = torch.zeros(0, 8, 64, device=DEV)
    lse = torch.zeros(0, 8, device=DEV)
    dst = torch.full((2, 0, 4, 64), 3.0, device=DEV)
    ops.dcp_pack_a2a_send(out, lse, dst, torch.zeros(2, 0, 4, device=DEV))
    torch.cuda.synchronize()


def test_pack_deterministic_and_repeatable():
    w, inp = inputs("longctx", 8)
    dt = w.dtype
    shape = (w.N, w.N, w.B, w.Hpr, w.D + 2)
    o = to_dev(inp["out"], dt, DEV)
    l = torch.from_numpy(inp["lse"]).to(DEV)
    res = []
    for _ in range(2):
        send = torch.zeros(shape, dtype=TORCH_DT[dt], device=DEV)
        pay, words = ops.interleaved_views(send, w.D)
        ops.dcp_pack_a2a_send(o, l, pay, words)
        res.append(send.view(torch.uint8).cpu())
    assert torch.equal(res[0], res[1])
