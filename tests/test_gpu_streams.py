"""Calls keep no state and enqueue only on the caller's stream: two
independent decode layers issued concurrently on two streams, from one host
thread or from two, give, bit for bit, what they give one after the other on
one stream."""
import pytest
import torch

from lse_weighted_merge_dcp_amd import sim, synth

from helpers import say, to_dev

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def layer_inputs(key, B, shift):
    w = synth.WORKLOADS[key].with_batch(B)
    inp = synth.rank_inputs(w)
    src = to_dev(inp["out"], w.dtype, DEV)
    lse = torch.from_numpy(inp["lse"]).to(DEV) + shift
    st = sim.StackedInterleaved(w.N, w.B, w.H, w.D, src.dtype, DEV)
    out = torch.empty((w.N, w.B, w.Hpr, w.D), dtype=src.dtype, device=DEV)
    g = torch.empty((w.N, w.B, w.Hpr), dtype=torch.float32, device=DEV)
    return w, src, lse, st, out, g


def run_layer(w, src, lse, st, out, g):
    st.pack(src, lse)
    st.combine(is_lse_base_on_e=not w.base2, out=out, out_lse=g)


def test_concurrent_streams_match_sequential():
    say("two streams")
    a = layer_inputs("longctx", 64, 0.0)
    b = layer_inputs("longctx", 8, 1.5)
    c = layer_inputs("dsv3fp8", 16, 0.5)     # an fp8 layer behind b on the second stream
    run_layer(*a)
    run_layer(*b)
    run_layer(*c)
    torch.cuda.synchronize()
    bufs = [x[i] if i != 3 else x[3].send for x in (a, b, c) for i in (3, 4, 5)]
    ref = [t.clone() for t in bufs]
    for t in bufs:
        t.view(torch.uint8).zero_()
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for rep in range(3):
        with torch.cuda.stream(s1):
            run_layer(*a)
        with torch.cuda.stream(s2):
            run_layer(*b)
            run_layer(*c)
        torch.cuda.synchronize()
        got = bufs
        for x, y in zip(got, ref):
            assert torch.equal(x.view(torch.uint8), y.view(torch.uint8)), "concurrent run %d differs" % rep


def test_concurrent_host_threads_match_sequential():
    """Two host threads, each on a stream of its own, issue different decode
    layers through the library over and over at the same time (ctypes drops
    the interpreter lock during the calls, so the library's host code runs
    in both threads at once); each thread's last results equal the
    sequential ones bit for bit."""
    import threading

    say("two host threads")
    layers = [layer_inputs("dsv3", 16, 0.0), layer_inputs("longctx", 8, 1.5)]
    for x in layers:
        run_layer(*x)
    torch.cuda.synchronize()
    bufs = [[x[3].send, x[4], x[5]] for x in layers]
    ref = [[t.clone() for t in b] for b in bufs]
    for b in bufs:
        for t in b:
            t.view(torch.uint8).zero_()
    torch.cuda.synchronize()
    errors = []
    start = threading.Barrier(2)

    def work(i):
        try:
            s = torch.cuda.Stream(device=DEV)
            start.wait(timeout=60)
            with torch.cuda.stream(s):
                for _ in range(25):
                    run_layer(*layers[i])
            s.synchronize()
        except Exception as e:  # reported in the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=work, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    for b, r in zip(bufs, ref):
        for x, y in zip(b, r):
            assert torch.equal(x.view(torch.uint8), y.view(torch.uint8)), "a threaded run differs"
