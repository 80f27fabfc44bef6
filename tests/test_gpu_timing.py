"""dcp_time_next_call: timing events travel with the next call's kernel
dispatches, change nothing in its results, cover exactly one call, are
cleared by a call that launches nothing or is rejected, and are refused
while the stream is being captured."""
import numpy as np
import pytest
import torch

from lse_weighted_merge_dcp_amd import _lib, ops, timing
from oracle import oracle as orc

from helpers import check_lse, check_out, say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
N, B, H, D = 4, 64, 32, 512


def inputs(seed=0):
    rng = np.random.default_rng(seed)
    out = rng.normal(size=(B, H, D)).astype(np.float32)
    lse = rng.normal(0, 3, size=(B, H)).astype(np.float32)
    return out, lse, torch.from_numpy(out).to(DEV).to(torch.bfloat16), torch.from_numpy(lse).to(DEV)


def send_buffers():
    send = torch.zeros((N, B, H // N, D + 2), dtype=torch.bfloat16, device=DEV)
    return (send,) + ops.interleaved_views(send, D)


def test_timed_calls_match_untimed():
    say("timed calls")
    _, _, o, l = inputs()
    results = []
    for timed in (False, True):
        ev = [timing.Event() for _ in range(6)]
        send, pay, words = send_buffers()
        if timed:
            ops.time_next_call(ev[0], ev[1])
        ops.dcp_pack_a2a_send(o, l, pay, words)
        if timed:
            ops.time_next_call(ev[2], ev[3])
        comb, g = ops.dcp_lse_combine(pay, words, is_lse_base_on_e=True, return_lse=True)
        part = torch.stack([o.float() * (r + 1) for r in range(N)])
        lses = torch.stack([l - r for r in range(N)])
        if timed:
            ops.time_next_call(ev[4], ev[5])
        merged, gl = ops.cp_lse_combine_inplace(part, lses, return_lse=True)
        torch.cuda.synchronize()
        results.append([t.clone() for t in (send, comb, g, part, merged, gl)])
        if timed:
            for i in range(0, 6, 2):
                us = ev[i].elapsed_us(ev[i + 1])
                assert 0.0 < us < 1e5, us
    for x, y in zip(*results):
        assert torch.equal(x.view(torch.uint8), y.view(torch.uint8))


def test_timed_combine_matches_the_oracle():
    say("timed combine vs oracle")
    out, lse, o, l = inputs(1)
    send, pay, words = send_buffers()
    ops.dcp_pack_a2a_send(o, l, pay, words)
    s, e = timing.Event(), timing.Event()
    ops.time_next_call(s, e)
    comb, g = ops.dcp_lse_combine(pay, words, is_lse_base_on_e=True, return_lse=True)
    torch.cuda.synchronize()
    assert s.elapsed_us(e) > 0
    host = send.cpu().view(torch.int16).numpy().view(np.uint16)
    wp, ww = orc.interleaved_views_np(host, D, "bf16")
    ref, gr, mag, _ = orc.combine(wp, ww, "bf16", False)
    check_out(comb.float().cpu().numpy(), ref, mag, "bf16")
    check_lse(g.cpu().numpy(), gr)


def test_request_covers_one_call():
    say("one call")
    _, _, o, l = inputs()
    send, pay, words = send_buffers()
    s, e = timing.Event(), timing.Event()
    ops.time_next_call(s, e)
    ops.dcp_pack_a2a_send(o, l, pay, words)
    torch.cuda.synchronize()
    first = s.elapsed_us(e)
    for _ in range(3):
        ops.dcp_pack_a2a_send(o, l, pay, words)
    torch.cuda.synchronize()
    assert s.elapsed_us(e) == first


def test_call_without_launch_clears_request():
    say("zero-sized call")
    _, _, o, l = inputs()
    send, pay, words = send_buffers()
    s, e = timing.Event(), timing.Event()
    ops.time_next_call(s, e)
    ops.dcp_pack_a2a_send(o[:0], l[:0], pay[:, :0], words[:, :0])
    ops.dcp_pack_a2a_send(o, l, pay, words)
    torch.cuda.synchronize()
    with pytest.raises(RuntimeError):     # never recorded
        s.elapsed_us(e)


def test_rejected_call_clears_request():
    say("rejected call")
    _, _, o, l = inputs()
    send, pay, words = send_buffers()
    s, e = timing.Event(), timing.Event()
    ops.time_next_call(s, e)
    st = _lib.lib().dcp_pack(o.data_ptr(), 0, 0, 0, l.data_ptr(), 0, 0, 0,
                             pay.data_ptr(), 0, 0, 0, 0, words.data_ptr(), 0, 0, 0, 0,
                             None, 0, 0, 1, N, B, H, D, 7, None)
    assert _lib.STATUS[st] == "DCP_ERR_DTYPE"
    ops.dcp_pack_a2a_send(o, l, pay, words)
    torch.cuda.synchronize()
    with pytest.raises(RuntimeError):
        s.elapsed_us(e)


def test_timed_call_refused_during_capture():
    say("capture")
    _, _, o, l = inputs()
    send, pay, words = send_buffers()
    ops.dcp_pack_a2a_send(o, l, pay, words)
    torch.cuda.synchronize()
    want = send.clone()
    send.zero_()
    s, e = timing.Event(), timing.Event()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ops.time_next_call(s, e)
        with pytest.raises(_lib.DcpError, match="DCP_ERR_CAPTURE"):
            ops.dcp_pack_a2a_send(o, l, pay, words)
        ops.dcp_pack_a2a_send(o, l, pay, words)     # untimed: captured as usual
    torch.cuda.synchronize()
    for _ in range(2):
        send.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(send.view(torch.uint8), want.view(torch.uint8))
