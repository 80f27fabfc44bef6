"""Seeded random shapes and layouts against the oracle (hypothesis,
derandomized: every run tries the same cases).

Each operand is a view into a larger buffer of random bytes, with a random
memory order of its outer axes, random padding on every axis and a random
element offset (so rows are often not 4- or 16-byte aligned); D stays
contiguous.  The draws span the launch-shape choices of the library: the
flat-stream and the row-by-row pack (1, 2 or 4 rows per wave), the
row-per-wave and the short-row combine, the fixed-N and any-N paths, both
load orders, ragged last segments, R > 1, zero KV lengths and special
values.  The pack must reproduce the oracle byte for byte over the whole
destination buffers (bytes outside the views untouched); the combine and
in-place outputs must be within tolerance, and the bytes of their buffers
outside the output views untouched.
"""

import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from lse_weighted_merge_dcp_amd import ops
from oracle import oracle as orc

from helpers import NP_DT, TORCH_DT, check_lse, check_out, check_scaled, decode, say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
SETTINGS = dict(max_examples=48, derandomize=True, deadline=None, print_blob=True,
                suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])
DTS = ["f32", "f16", "bf16", "fp8"]
SPECIAL = np.array([np.nan, np.inf, -np.inf], np.float32)


class Buf:
    """A host buffer of random bytes and the same bytes on the device, with a
    strided view of `shape` into both."""

    def __init__(self, rng, shape, np_dt, torch_dt, last_contig=True):
        nd = len(shape)
        inner_axes = list(range(nd - 1)) if last_contig else list(range(nd))
        order = list(rng.permutation(inner_axes)) + ([nd - 1] if last_contig else [])   # outer -> inner
        pads = {a: int(rng.choice([0, 0, 1, 3])) for a in range(nd)}
        strides = [0] * nd
        extent = 1
        for a in reversed(order):
            strides[a] = extent
            extent *= shape[a] + pads[a]
        self.offset = int(rng.integers(0, 4))
        total = self.offset + max(extent, 1)
        itemsize = np.dtype(np_dt).itemsize
        self.host = np.frombuffer(rng.bytes(total * itemsize), np_dt).copy()
        self.shape, self.strides, self.np_dt, self.torch_dt = tuple(shape), tuple(strides), np_dt, torch_dt
        self.dev = None

    def hview(self):
        it = self.host.itemsize
        return np.lib.stride_tricks.as_strided(self.host[self.offset:], self.shape, [s * it for s in self.strides],
                                               writeable=True)

    def upload(self):
        h = self.host
        if self.np_dt == np.uint16:
            self.dev = torch.from_numpy(h.view(np.int16)).to(DEV).view(torch.bfloat16)
        elif self.np_dt == np.uint8 and self.torch_dt == torch.float8_e4m3fn:
            self.dev = torch.from_numpy(h).to(DEV).view(torch.float8_e4m3fn)
        else:
            self.dev = torch.from_numpy(h).to(DEV)
        return self

    def dview(self):
        return torch.as_strided(self.dev, self.shape, self.strides, self.offset)

    def download(self):
        t = self.dev.cpu()
        if self.np_dt == np.uint16:
            return t.view(torch.int16).numpy().view(np.uint16)
        if t.dtype == torch.float8_e4m3fn:
            return t.view(torch.uint8).numpy()
        return t.numpy()


def payload_buf(rng, shape, dt):
    return Buf(rng, shape, NP_DT[dt], TORCH_DT[dt])


def lse_buf(rng, shape):
    return Buf(rng, shape, np.float32, torch.float32, last_contig=False)


def fill_payload(rng, buf, dt, specials):
    """Normal values (with NaN/inf sprinkled if specials) into the view."""
    x = rng.normal(size=buf.shape).astype(np.float32)
    if specials and x.size:
        idx = rng.integers(0, x.size, size=max(1, x.size // 200))
        x.reshape(-1)[idx] = SPECIAL[rng.integers(0, 3, size=idx.size)]
    v = buf.hview()
    if dt == "bf16":
        b = x.view(np.uint32)
        r = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)     # round to nearest even
        r[np.isnan(x)] = 0x7FC0
        v[...] = r
    elif dt == "fp8":
        v[...] = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()   # inf becomes NaN
    else:
        v[...] = x.astype(NP_DT[dt])


def fill_lse(rng, buf, specials):
    l = rng.normal(0, 4, size=buf.shape).astype(np.float32)
    if l.size:
        l.reshape(-1)[rng.integers(0, l.size, size=max(1, l.size // 10))] = -np.inf
        if specials:
            idx = rng.integers(0, l.size, size=max(1, l.size // 50))
            l.reshape(-1)[idx] = SPECIAL[rng.integers(0, 3, size=idx.size)]
    buf.hview()[...] = l


def outside_unchanged(buf, got):
    """The downloaded buffer equals the original host bytes outside the view."""
    mask = np.ones(buf.host.shape, bool)
    idx = np.zeros(buf.shape, np.int64)
    for a, (n, s) in enumerate(zip(buf.shape, buf.strides)):
        sh = [1] * len(buf.shape)
        sh[a] = n
        idx = idx + (np.arange(n, dtype=np.int64) * s).reshape(sh)
    mask[buf.offset + idx.reshape(-1)] = False
    assert np.array_equal(got[mask].view(np.uint8), buf.host[mask].view(np.uint8)), "bytes outside the view changed"


@settings(**SETTINGS)
@given(st.data())
def test_fuzz_pack(data):
    dt = data.draw(st.sampled_from(DTS))
    N = data.draw(st.sampled_from([1, 2, 3, 4, 8, 16]))
    Hpr = data.draw(st.integers(1, 9))
    H = N * Hpr
    lpd = 4 // np.dtype(NP_DT[dt]).itemsize
    interleaved = data.draw(st.booleans())
    if interleaved:
        D = lpd * data.draw(st.sampled_from([1, 3, 32, 64, 255, 256, 300, 512]))
    else:
        D = data.draw(st.sampled_from([1, 2, 7, 64, 100, 128, 512, 600]))
    B = data.draw(st.integers(0, 9))
    R = data.draw(st.integers(1, 3))
    use_kv = data.draw(st.booleans())
    seed = data.draw(st.integers(0, 2 ** 31 - 1))
    rng = np.random.default_rng(seed)
    say("fuzz pack", dt, "N", N, "Hpr", Hpr, "D", D, "B", B, "R", R, "interleaved", interleaved, "kv", use_kv, "seed", seed)

    src = payload_buf(rng, (R, B, H, D), dt)           # random bits: the pack is a bit copy
    lse = lse_buf(rng, (R, B, H))
    kv = rng.integers(0, 3, size=(R, B)).astype(np.int32) if use_kv else None
    if interleaved:
        send = np.frombuffer(rng.bytes(R * N * B * Hpr * (D + lpd) * np.dtype(NP_DT[dt]).itemsize),
                             NP_DT[dt]).reshape(R, N, B, Hpr, D + lpd).copy()
        d_send = torch.from_numpy(send.view(np.int16) if dt == "bf16" else send).to(DEV)
        if dt in ("bf16", "fp8"):
            d_send = d_send.view(TORCH_DT[dt])
        d_pay, d_words = ops.interleaved_views(d_send, D)
        ops.dcp_pack_a2a_send(src.upload().dview(), lse.upload().dview(), d_pay, d_words,
                              kv_len=torch.from_numpy(kv).to(DEV) if use_kv else None)
        got = d_send.cpu()
        got = got.view(torch.int16).numpy().view(np.uint16) if dt == "bf16" else got.view(torch.uint8).numpy() \
            if dt == "fp8" else got.numpy()
        want = send.copy()
        h_pay, h_words = orc.interleaved_views_np(want, D, dt)
        for r in range(R):
            orc.pack(src.hview()[r], lse.hview()[r], h_pay[r], h_words[r], N, kv_len=kv[r] if use_kv else None)
        assert np.array_equal(got.view(np.uint8), want.view(np.uint8))
    else:
        dst = payload_buf(rng, (R, N, B, Hpr, D), dt)
        dst_l = lse_buf(rng, (R, N, B, Hpr))
        ops.dcp_pack_a2a_send(src.upload().dview(), lse.upload().dview(), dst.upload().dview(), dst_l.upload().dview(),
                              kv_len=torch.from_numpy(kv).to(DEV) if use_kv else None)
        got_o, got_l = dst.download(), dst_l.download()
        for r in range(R):
            orc.pack(src.hview()[r], lse.hview()[r], dst.hview()[r], dst_l.hview()[r], N,
                     kv_len=kv[r] if use_kv else None)
        assert np.array_equal(got_o.view(np.uint8), dst.host.view(np.uint8))
        assert np.array_equal(got_l.view(np.uint8), dst_l.host.view(np.uint8))


@settings(**SETTINGS)
@given(st.data())
def test_fuzz_combine(data):
    dt = data.draw(st.sampled_from(DTS))
    N = data.draw(st.sampled_from([1, 2, 3, 4, 5, 8, 16, 17, 33]))
    Hpr = data.draw(st.integers(1, 9))
    D = data.draw(st.sampled_from([1, 8, 63, 64, 128, 384, 400, 512, 520, 1000]))
    B = data.draw(st.integers(0, 40))
    R = data.draw(st.integers(1, 2))
    base2 = data.draw(st.booleans())
    specials = data.draw(st.booleans())
    want_lse = data.draw(st.booleans())
    seed = data.draw(st.integers(0, 2 ** 31 - 1))
    rng = np.random.default_rng(seed)
    say("fuzz combine", dt, "N", N, "Hpr", Hpr, "D", D, "B", B, "R", R, "base2", base2, "specials", specials, "seed", seed)

    recv = payload_buf(rng, (R, N, B, Hpr, D), dt)
    fill_payload(rng, recv, dt, specials)
    rl = lse_buf(rng, (R, N, B, Hpr))
    fill_lse(rng, rl, specials)
    out = payload_buf(rng, (R, B, Hpr, D), dt).upload()
    out_l = lse_buf(rng, (R, B, Hpr)).upload()
    ops.dcp_lse_combine(recv.upload().dview(), rl.upload().dview(), is_lse_base_on_e=not base2,
                        return_lse=want_lse, out=out.dview(), out_lse=out_l.dview() if want_lse else None)
    got_o = out.download()
    outside_unchanged(out, got_o)
    got_l = out_l.download()
    if not want_lse:
        assert np.array_equal(got_l.view(np.uint8), out_l.host.view(np.uint8))
    else:
        outside_unchanged(out_l, got_l)
    ov = np.lib.stride_tricks.as_strided(got_o[out.offset:], out.shape, [s * got_o.itemsize for s in out.strides])
    lv = np.lib.stride_tricks.as_strided(got_l[out_l.offset:], out_l.shape, [s * 4 for s in out_l.strides])
    for r in range(R):
        if N == 1:      # identity, bit for bit
            assert np.array_equal(np.ascontiguousarray(ov[r]).view(np.uint8),
                                  np.ascontiguousarray(recv.hview()[r, 0]).view(np.uint8))
            if want_lse:
                assert np.array_equal(np.ascontiguousarray(lv[r]).view(np.uint32),
                                      np.ascontiguousarray(rl.hview()[r, 0]).view(np.uint32))
            continue
        ref, gr, mag, _ = orc.combine(np.ascontiguousarray(recv.hview()[r]), np.ascontiguousarray(rl.hview()[r]), dt, base2)
        check_out(decode(np.ascontiguousarray(ov[r]), dt), ref, mag, dt, "r=%d" % r)
        if want_lse:
            check_lse(np.ascontiguousarray(lv[r]), gr)


@settings(**SETTINGS)
@given(st.data())
def test_fuzz_inplace(data):
    dt = data.draw(st.sampled_from(DTS))
    N = data.draw(st.sampled_from([1, 2, 3, 4, 8, 16, 17]))
    P = data.draw(st.integers(1, N))
    rank0 = data.draw(st.integers(0, N - P))
    H = data.draw(st.integers(1, 12))
    h0 = data.draw(st.integers(0, H - 1))
    h1 = data.draw(st.integers(h0 + 1, H))
    D = data.draw(st.sampled_from([1, 8, 64, 100, 256, 512, 520]))
    T = data.draw(st.integers(0, 24))
    base2 = data.draw(st.booleans())
    specials = data.draw(st.booleans())
    want_out = data.draw(st.booleans())
    seed = data.draw(st.integers(0, 2 ** 31 - 1))
    rng = np.random.default_rng(seed)
    say("fuzz inplace", dt, "N", N, "P", P, "rank0", rank0, "H", H, "h", h0, h1, "D", D, "T", T, "base2", base2,
        "seed", seed)

    part = payload_buf(rng, (P, T, H, D), dt)
    fill_payload(rng, part, dt, specials)
    lse = lse_buf(rng, (N, T, H))
    fill_lse(rng, lse, specials)
    out = payload_buf(rng, (T, h1 - h0, D), dt)
    out_l = lse_buf(rng, (T, h1 - h0))
    before = np.ascontiguousarray(part.hview()).copy()
    res = ops.cp_lse_combine_inplace(part.upload().dview(), lse.upload().dview(), h0=h0, h1=h1, rank0=rank0,
                                     is_lse_base_on_e=not base2, return_lse=True,
                                     out=out.upload().dview() if want_out else None,
                                     out_lse=out_l.upload().dview(), want_out=want_out)
    torch.cuda.synchronize()
    got_p = part.download()
    outside_unchanged(part, got_p)
    pv = np.lib.stride_tricks.as_strided(got_p[part.offset:], part.shape, [s * got_p.itemsize for s in part.strides])
    got_l = out_l.download()
    outside_unchanged(out_l, got_l)
    lv = np.lib.stride_tricks.as_strided(got_l[out_l.offset:], out_l.shape, [s * 4 for s in out_l.strides])
    scaled, ref, gr, mag = orc.inplace(before, np.ascontiguousarray(lse.hview()), dt, base2, rank0=rank0, h0=h0, h1=h1)
    if N == 1:
        assert np.array_equal(np.ascontiguousarray(pv).view(np.uint8), before.view(np.uint8))
    else:
        check_scaled(decode(np.ascontiguousarray(pv), dt), scaled, dt)
    if want_out:
        got_o = out.download()
        outside_unchanged(out, got_o)
        ov = np.lib.stride_tricks.as_strided(got_o[out.offset:], out.shape, [s * got_o.itemsize for s in out.strides])
        if N == 1:
            assert np.array_equal(np.ascontiguousarray(ov).view(np.uint8),
                                  np.ascontiguousarray(before[0][:, h0:h1]).view(np.uint8))
        else:
            check_out(decode(np.ascontiguousarray(ov), dt), ref, mag, dt)
    if N == 1:
        assert np.array_equal(np.ascontiguousarray(lv).view(np.uint32),
                              np.ascontiguousarray(lse.hview()[0][:, h0:h1]).view(np.uint32))
    else:
        check_lse(np.ascontiguousarray(lv), gr)
