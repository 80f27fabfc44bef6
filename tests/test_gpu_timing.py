"""Timed calls (libdcpmerge_bench.so, reached through ops' timing=(start,
stop)): the events travel with the call's own kernel dispatches, change
nothing in its results, are left unrecorded by a call that launches nothing
or is rejected, and are refused while the stream is being captured.  Calls
without events go to libdcpmerge.so, which takes no events at all."""
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
        tm = [(ev[i], ev[i + 1]) if timed else None for i in (0, 2, 4)]
        send, pay, words = send_buffers()
        ops.dcp_pack_a2a_send(o, l, pay, words, timing=tm[0])
        comb, g = ops.dcp_lse_combine(pay, words, is_lse_base_on_e=True, return_lse=True, timing=tm[1])
        part = torch.stack([o.float() * (r + 1) for r in range(N)])
        lses = torch.stack([l - r for r in range(N)])
        merged, gl = ops.cp_lse_combine_inplace(part, lses, return_lse=True, timing=tm[2])
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
    comb, g = ops.dcp_lse_combine(pay, words, is_lse_base_on_e=True, return_lse=True, timing=(s, e))
    torch.cuda.synchronize()
    assert s.elapsed_us(e) > 0
    host = send.cpu().view(torch.int16).numpy().view(np.uint16)
    wp, ww = orc.interleaved_views_np(host, D, "bf16")
    ref, gr, mag, _ = orc.combine(wp, ww, "bf16", False)
    check_out(comb.float().cpu().numpy(), ref, mag, "bf16")
    check_lse(g.cpu().numpy(), gr)


def test_start_or_stop_alone():
    say("one event")
    _, _, o, l = inputs()
    send, pay, words = send_buffers()
    a, b = timing.Event(), timing.Event()
    ops.dcp_pack_a2a_send(o, l, pay, words, timing=(a, None))
    ops.dcp_pack_a2a_send(o, l, pay, words, timing=(None, b))
    torch.cuda.synchronize()
    assert a.elapsed_us(b) > 0


def test_launch_shape_of_a_call():
    """A call given a shape record reports what it launched; an empty
    kernel of that shape runs."""
    say("launch shape")
    _, _, o, l = inputs()
    send, pay, words = send_buffers()
    shape = timing.LaunchShape()
    ops.dcp_pack_a2a_send(o, l, pay, words, timing=(None, None, shape))
    assert shape.launches == 1 and shape.blocks >= 1 and shape.threads in (64, 128, 256, 512)
    timing.empty_kernel(shape.blocks, shape.threads, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()


def test_call_without_launch_records_nothing():
    say("zero-sized call")
    _, _, o, l = inputs()
    send, pay, words = send_buffers()
    s, e = timing.Event(), timing.Event()
    ops.dcp_pack_a2a_send(o[:0], l[:0], pay[:, :0], words[:, :0], timing=(s, e))
    ops.dcp_pack_a2a_send(o, l, pay, words)
    torch.cuda.synchronize()
    with pytest.raises(RuntimeError):     # never recorded
        s.elapsed_us(e)


def test_rejected_call_records_nothing():
    say("rejected call")
    _, _, o, l = inputs()
    send, pay, words = send_buffers()
    s, e = timing.Event(), timing.Event()
    st = timing.bench_lib().dcpb_pack(s.handle, e.handle, o.data_ptr(), 0, 0, 0, l.data_ptr(), 0, 0, 0,
                                      pay.data_ptr(), 0, 0, 0, 0, words.data_ptr(), 0, 0, 0, 0,
                                      None, 0, 0, 1, N, B, H, D, 7, None, None)
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
        with pytest.raises(timing.CaptureError, match="DCPB_ERR_CAPTURE"):
            ops.dcp_pack_a2a_send(o, l, pay, words, timing=(s, e))
        ops.dcp_pack_a2a_send(o, l, pay, words)     # untimed: captured as usual
    torch.cuda.synchronize()
    for _ in range(2):
        send.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(send.view(torch.uint8), want.view(torch.uint8))
