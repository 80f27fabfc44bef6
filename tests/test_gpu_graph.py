"""The library enqueues only kernels on the caller's stream (no allocation,
no memset, no host sync), so a whole multi-layer step can be captured in a
HIP graph.  Replays, with eager work and synchronisations between them, must
reproduce the eager result bit for bit."""
import pytest
import torch

from lse_weighted_merge_dcp_amd import ops, sim, synth

from helpers import say, to_dev

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def test_graph_replays_match_eager():
    w = synth.WORKLOADS["longctx"].with_batch(8)
    inp = synth.rank_inputs(w)
    say("graph", w.describe())
    L = 4
    src = [to_dev(inp["out"], w.dtype, DEV) for _ in range(L)]
    lse = [torch.from_numpy(inp["lse"]).to(DEV) + l for l in range(L)]
    stk = [sim.StackedInterleaved(w.N, w.B, w.H, w.D, torch.bfloat16, DEV) for _ in range(L)]
    outs = [torch.empty((w.N, w.B, w.Hpr, w.D), dtype=torch.bfloat16, device=DEV) for _ in range(L)]
    gl = [torch.empty((w.N, w.B, w.Hpr), dtype=torch.float32, device=DEV) for _ in range(L)]
    w8 = synth.WORKLOADS["dsv3fp8"].with_batch(4)          # an fp8 layer in the same step
    inp8 = synth.rank_inputs(w8)
    src8 = to_dev(inp8["out"], w8.dtype, DEV)
    lse8 = torch.from_numpy(inp8["lse"]).to(DEV)
    stk8 = sim.StackedInterleaved(w8.N, w8.B, w8.H, w8.D, torch.float8_e4m3fn, DEV)
    out8 = torch.empty((w8.N, w8.B, w8.Hpr, w8.D), dtype=torch.float8_e4m3fn, device=DEV)
    part = torch.randn(8, 16, 12, 128, device=DEV)
    plse = torch.randn(8, 16, 12, device=DEV)
    pcopy = part.clone()
    pout = torch.empty(16, 12, 128, device=DEV)

    def step():
        for l in range(L):
            stk[l].pack(src[l], lse[l])
            stk[l].combine(is_lse_base_on_e=False, out=outs[l], out_lse=gl[l])
        stk8.pack(src8, lse8)
        stk8.combine(is_lse_base_on_e=False, out=out8)
        ops.cp_lse_combine_inplace(part, plse, out=pout)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs] + [g.clone() for g in gl] + [pout.clone(), part.clone(), out8.view(torch.uint8).clone()]
    g = torch.cuda.CUDAGraph()
    for o in outs:
        o.zero_()
    part.copy_(pcopy)
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for o in outs:
            o.fill_(7.0)
        pout.zero_()
        out8.view(torch.uint8).fill_(0x38)
        part.copy_(pcopy)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = outs + gl + [pout, part, out8]
        for a, b in zip(got, ref):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), "replay %d differs" % rep
