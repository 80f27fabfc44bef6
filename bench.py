"""Benchmark of the DCP partial-merge path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload dsv3|longctx|split|tiny|kimi|kimi-rs|dsv3fp8] [--B 64]

Default run: the long-context decode sweep at B = 512 -- N=16 simulated DCP
ranks, 512 tokens, H=128 heads (8 per rank), D=512 bf16 partials, fp32
base-2 LSE, per-rank KV lengths uniform 0..64K (a rank with none holds the
neutral pair), peer-outer interleaved send buffers [N,B,8,514].  One step is
one decode step over 61 MLA layers; each layer packs all 16 ranks' send
buffers (one launch) and combines all 16 destinations (one launch), the
exchange between them being a zero-copy view of the stacked send buffers.
The layers rotate over distinct buffer sets (at least four, and at least
2 GiB of them), so no
layer's inputs are cache-resident when it runs.  The step is captured once
in a HIP graph and replayed K times; inputs are in HBM before timing
starts.  The DeepSeek-V3-shaped decode (N=8, B=64, H=128, D=512 bf16) and
the Kimi-K3-shaped in-place merge are measured after it and reported under
"secondary".

Printed: one JSON line with the whole-step throughput in GB/s of algorithmic
bytes (what the method must move: (3N+1)(D*e+4) bytes per (token, head) for
pack + combine), microseconds per layer, the roofline entry of the dominant
kernel (its per-launch duration inside the step, from HIP events attached to
its own dispatches in eager replays of the step; the same kernel's launches
replayed back to back on cold buffers give `cold_achieved`) and the CPU
oracle timed on a bounded sample, on every host thread and on one.  Beside
them: the p10/p50/p90 step time, the rate of a plain 2 GiB device-to-device
copy measured in the same run (the practical ceiling), for every kernel a
plain copy of the same size timed cold the same way (`copy_same_bytes`: the
rate a copy reaches at that size, fixed costs included), and for the pack +
combine workloads the per-rank share (one rank's pack and one destination's
combine at their real shapes, against the empty-kernel floor of their launch
shape and a same-size copy) and the cache-resident step (one layer's
buffers reused by every layer).

Other workloads: longctx (N=16, H=128, bf16, --B 1..512), split (peer-inside
split layout, fp16), tiny (N=2 fp32), kimi (in-place merge over 8 ranks'
[16384, 96, 512] fp32 partials), kimi-rs (the same merge, reduce-scatter
flavour: each rank's head slice, no partial write-back), dsv3fp8 (the
DeepSeek-V3 shape with an OCP FP8 E4M3 payload: rows of D + 4 bytes).

Other modes:
  --counter-run       run a 1 GiB plain copy and three calls of each kernel,
                      each timed (the command to put under rocprofv3 --pmc)
  --summarize-counters DIR[,DIR]   turn the rocprofv3 counter CSVs found in
                      the directories into profiles/counters_<workload>.json
  --summarize-spread GLOB   counter-run logs of fresh processes (plain or
                      under a counter pass) -> profiles/spread_<workload>.json
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0   # MI355X HBM3E, 8 TB/s
METRIC = "pack+LSE-combine HBM GB/s (% of MI355X peak); µs per MLA layer decode step"
CSRC = os.path.join(ROOT, "lse_weighted_merge_dcp_amd", "csrc")


def kernel_source_hash() -> str:
    """Hash of the library's sources with comments and blank lines removed:
    it changes when the code changes, not when a comment does."""
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.hpp"))
                    + glob.glob(os.path.join(CSRC, "*.cpp"))):
        text = open(p).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update("\n".join(line.rstrip() for line in text.splitlines() if line.strip()).encode())
    return h.hexdigest()[:16]


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------
def algorithmic_bytes(key, B=None):
    """Bytes each kernel of a workload must move per launch (what the method
    itself reads and writes; no re-reads):
      pack     2 N B H (D e + 4)     every rank reads and writes its rows
      combine  (N + 1) B H (D e + 4) N partial rows read, out + G written
      inplace  T H (N (4D + 4) + N 4D + 4D + 4)
      kimi-rs combine  T H (N (4D + 4) + 4D + 4)
    and, for the Kimi-K3 workloads, one rank's own call in a real group:
      inplace_rank  T H (2 4D + 4N)         scale its partial (P = 1)
      combine_rank  T H/N (N (4D + 4) + 4D + 4)   its head slice."""
    from lse_weighted_merge_dcp_amd import synth

    w = synth.WORKLOADS["kimi" if key == "kimi-rs" else key]
    if B is not None:
        w = w.with_batch(B)
    if key == "kimi":
        row = 4 * w.D
        return {"inplace": w.B * w.H * (w.N * (row + 4) + w.N * row + row + 4),
                "inplace_rank": w.B * w.H * (2 * row + 4 * w.N)}
    if key == "kimi-rs":
        row = 4 * w.D
        return {"combine": w.B * w.H * (w.N * (row + 4) + row + 4),
                "combine_rank": w.B * (w.H // w.N) * (w.N * (row + 4) + row + 4)}
    row = w.D * w.esize + 4
    per_th = w.B * w.H
    return {"pack": 2 * w.N * per_th * row, "combine": (w.N + 1) * per_th * row}


class A2AWorkload:
    """Interleaved or split pack + combine, `layers` distinct buffer sets."""

    def __init__(self, key, B, layers, dev, kv=False):
        import numpy as np
        import torch

        from lse_weighted_merge_dcp_amd import sim, synth

        w = synth.WORKLOADS[key]
        if B is not None:
            w = w.with_batch(B)
        self.w, self.layers, self.dev = w, layers, dev
        tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16,
               "fp8": torch.float8_e4m3fn}[w.dtype]
        t0 = time.time()
        self.inp = synth.rank_inputs(w)
        print("# generated %s in %.1f s" % (w.describe(), time.time() - t0), file=sys.stderr, flush=True)
        o = self.inp["out"]
        if w.dtype == "bf16":
            o0 = torch.from_numpy(o.view(np.int16)).to(dev).view(torch.bfloat16)
        elif w.dtype == "fp8":
            o0 = torch.from_numpy(o).to(dev).view(torch.float8_e4m3fn)
        else:
            o0 = torch.from_numpy(o).to(dev)
        l0 = torch.from_numpy(self.inp["lse"]).to(dev)
        # with kv: the pack reads each rank's KV length per token and sends the
        # neutral pair itself where it is 0 (interleaved workloads only)
        self.kv = None
        if kv:
            if w.layout != "interleaved" or self.inp["kv_len"] is None:
                raise SystemExit("--kv-len needs a workload with per-rank KV lengths (dsv3, longctx, dsv3fp8)")
            self.kv = torch.from_numpy(self.inp["kv_len"].astype(np.int32)).to(dev)
        self.src, self.lse, self.stk, self.out, self.glse = [], [], [], [], []
        cls = sim.StackedSplit if w.layout == "split" else sim.StackedInterleaved
        # distinct buffer sets: one per layer while that stays under 16 GiB, else
        # enough sets rotated that >= 2 GiB of other traffic separates two uses
        per_layer = 2 * o0.numel() * o0.element_size() + w.N * w.B * w.Hpr * w.D * o0.element_size()
        if per_layer * layers <= (16 << 30):
            self.distinct = layers
        else:
            self.distinct = min(layers, max(4, math.ceil((2 << 30) / per_layer)))
        for _ in range(self.distinct):
            self.src.append(o0.clone())
            self.lse.append(l0.clone())
            st = cls(w.N, w.B, w.H, w.D, tdt, dev)
            self.stk.append(st)
            self.out.append(torch.empty((w.N, w.B, w.Hpr, w.D), dtype=tdt, device=dev))
            self.glse.append(torch.empty((w.N, w.B, w.Hpr), dtype=torch.float32, device=dev))
        if w.layout == "split":
            # the exchange is a collective, not part of the merge: run it once, untimed
            for l in range(self.distinct):
                self.stk[l].pack(self.src[l], self.lse[l])
                self.stk[l].exchange()
        torch.cuda.synchronize()
        nb = algorithmic_bytes(key, B)
        self.bytes_pack, self.bytes_combine = nb["pack"], nb["combine"]
        self.bytes_layer = self.bytes_pack + self.bytes_combine

    def pack(self, l, timing=None):
        k = l % self.distinct
        self.stk[k].pack(self.src[k], self.lse[k], kv_len=self.kv, timing=timing)

    def combine(self, l, timing=None):
        k = l % self.distinct
        self.stk[k].combine(is_lse_base_on_e=not self.w.base2, out=self.out[k], out_lse=self.glse[k],
                            timing=timing)

    def pack_rank0(self, l, timing=None):
        k = l % self.distinct
        self.stk[k].pack_rank(0, self.src[k][0], self.lse[k][0], kv_len=None if self.kv is None else self.kv[0],
                              timing=timing)

    def combine_dest0(self, l, timing=None):
        k = l % self.distinct
        self.stk[k].combine_dest(0, not self.w.base2, out=self.out[k][0], out_lse=self.glse[k][0], timing=timing)

    def per_rank(self):
        """One rank's pack and one destination's combine at their real shapes
        (1/N of the all-rank launches), over the same distinct layer buffers."""
        N = self.w.N
        return [("pack", self.bytes_pack // N, [lambda l=l, **kw: self.pack_rank0(l, **kw) for l in range(self.layers)]),
                ("combine", self.bytes_combine // N,
                 [lambda l=l, **kw: self.combine_dest0(l, **kw) for l in range(self.layers)])]

    def hot_launches(self):
        """The step with one layer's buffers reused by every layer (cache-resident)."""
        fns = []
        for _ in range(self.layers):
            fns.append(lambda: self.pack(0))
            fns.append(lambda: self.combine(0))
        return fns

    def step_launches(self):
        return [f for _, f in self.named_step()]

    def named_step(self):
        """The step's calls in order, each with the kernel it launches."""
        fns = []
        for l in range(self.layers):
            fns.append(("pack", lambda l=l, **kw: self.pack(l, **kw)))
            fns.append(("combine", lambda l=l, **kw: self.combine(l, **kw)))
        return fns

    def kernels(self):
        """(name, per-launch algorithmic bytes, list of launch closures)."""
        return [("pack", self.bytes_pack, [lambda l=l, **kw: self.pack(l, **kw) for l in range(self.layers)]),
                ("combine", self.bytes_combine,
                 [lambda l=l, **kw: self.combine(l, **kw) for l in range(self.layers)])]

    def step_bytes(self):
        return self.layers * self.bytes_layer

    def config(self):
        w = self.w
        return {"workload": "%s: N=%d simulated ranks, B=%d, H=%d (%d per rank), D=%d %s, base-%s LSE, %s layout, "
                            "%d layers per step" % (
                                {"dsv3": "DeepSeek-V3-shaped MLA decode", "longctx": "long-context decode sweep",
                                 "split": "peer-inside split layout", "tiny": "tiny merge",
                                 "dsv3fp8": "DeepSeek-V3-shaped MLA decode, fp8 payload"}[w.key],
                                w.N, w.B, w.H, w.Hpr, w.D, w.dtype, "2" if w.base2 else "e", w.layout,
                                self.layers),
                "N": w.N, "B": w.B, "H": w.H, "D": w.D, "payload_dtype": w.dtype, "layers": self.layers,
                "layout": w.layout, "kv_len_in_pack": self.kv is not None,
                "distinct_buffer_sets": self.distinct}

    def cpu_sample(self, budget_s):
        """Time the oracle on whole layers of the same workload (pack of every rank
        and combine of every destination, interleaved layout) within ~budget_s."""
        import numpy as np

        from oracle import oracle as orc

        w, inp = self.w, self.inp
        lpd = 4 // w.esize
        npdt = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16, "fp8": np.uint8}[w.dtype]
        done, t_total = 0, 0.0
        while True:
            t0 = time.perf_counter()
            send = np.empty((w.N, w.N, w.B, w.Hpr, w.D + lpd), npdt)
            pay, words = orc.interleaved_views_np(send, w.D, w.dtype)
            for r in range(w.N):
                kv = None if self.kv is None else np.ascontiguousarray(inp["kv_len"][r], np.int32)
                orc.pack(inp["out"][r], inp["lse"][r], pay[r], words[r], w.N, kv_len=kv)
            for p in range(w.N):
                orc.combine(pay[:, p], words[:, p], w.dtype, w.base2)
            t_total += time.perf_counter() - t0
            done += 1
            if t_total >= budget_s:
                break
        return {"value": self.bytes_layer * done / t_total / 1e9, "unit": "GB/s", "cores": orc.num_threads(),
                "kind": "oracle",
                "sample": "%d whole layer(s) of the same workload (pack of all %d ranks + combine of all %d "
                          "destinations), %.1f s of CPU time, fp64" % (done, w.N, w.N, t_total),
                "us_per_layer": t_total / done * 1e6}


class InplaceWorkload:
    """The in-place merge over every rank's partial (Kimi-K3 cached-extend shape)."""

    def __init__(self, B, dev):
        import torch

        from lse_weighted_merge_dcp_amd import synth

        w = synth.WORKLOADS["kimi"]
        if B is not None:
            w = w.with_batch(B)
        self.w, self.dev, self.layers = w, dev, 1
        t0 = time.time()
        self.part = synth.kimi_partial_device(w, dev)
        self.pristine = self.part.clone()
        self.lse_np = synth.kimi_lse(w)
        self.lse = torch.from_numpy(self.lse_np).to(dev)
        self.out = torch.empty((w.B, w.H, w.D), dtype=torch.float32, device=dev)
        self.glse = torch.empty((w.B, w.H), dtype=torch.float32, device=dev)
        torch.cuda.synchronize()
        print("# generated %s in %.1f s" % (w.describe(), time.time() - t0), file=sys.stderr, flush=True)
        self.bytes_call = algorithmic_bytes("kimi", B)["inplace"]

    def run(self, timing=None):
        from lse_weighted_merge_dcp_amd import ops

        ops.cp_lse_combine_inplace(self.part, self.lse, out=self.out, out_lse=self.glse, return_lse=True,
                                   timing=timing)

    def restore(self):
        self.part.copy_(self.pristine)

    def kernels(self):
        return [("inplace", self.bytes_call, [self.run])]

    def per_rank(self):
        """What one GPU of a real DCP group runs: its own call (P = 1) that
        scales its partial [T, H, D] in place by its weight from all N LSEs;
        the sum over ranks is then the collective's.  Bytes: the partial read
        and written back, and the N LSEs of every (token, head)."""
        from lse_weighted_merge_dcp_amd import ops

        nbytes = algorithmic_bytes("kimi", self.w.B)["inplace_rank"]

        def call(timing=None):
            ops.cp_lse_combine_inplace(self.part[0:1], self.lse, rank0=0, want_out=False, timing=timing)

        return [("inplace", nbytes, [call])]

    def named_step(self):
        return [("inplace", self.run)]

    def step_bytes(self):
        return self.bytes_call

    def config(self):
        w = self.w
        return {"workload": "Kimi-K3-shaped cached-extend in-place merge: N=8 ranks' partials [%d, %d, %d] fp32, "
                            "base-e LSE with 0.1%% NaN/inf" % (w.B, w.H, w.D),
                "N": w.N, "T": w.B, "H": w.H, "D": w.D, "payload_dtype": "f32"}

    def cpu_sample(self, budget_s):
        import numpy as np

        from oracle import oracle as orc

        w = self.w
        tblk = 64
        done, t_total = 0, 0.0
        while t_total < budget_s and done + tblk <= w.B:
            part = self.pristine[:, done:done + tblk].cpu().numpy()
            lse = self.lse_np[:, done:done + tblk]
            t0 = time.perf_counter()
            orc.inplace(part, lse, "f32", False)
            t_total += time.perf_counter() - t0
            done += tblk
        per_tok = self.bytes_call / w.B
        return {"value": per_tok * done / t_total / 1e9, "unit": "GB/s", "cores": orc.num_threads(), "kind": "oracle",
                "sample": "first %d of %d tokens (all 8 ranks, 96 heads), %.1f s of CPU time, fp64" % (
                    done, w.B, t_total)}


class ReduceScatterWorkload:
    """Reduce-scatter flavour of the in-place merge (Kimi-K3 cached-extend
    shape): every rank's head slice of the merged output straight from all N
    partials, with no write-back of scaled partials.  The N ranks' slices
    tile the heads, so their out-of-place combines run as one combine over
    all heads of the partial stack (sim.reduce_scatter_merge)."""

    def __init__(self, B, dev):
        import torch

        from lse_weighted_merge_dcp_amd import synth

        w = synth.WORKLOADS["kimi"]
        if B is not None:
            w = w.with_batch(B)
        self.w, self.dev, self.layers = w, dev, 1
        t0 = time.time()
        self.part = synth.kimi_partial_device(w, dev)
        self.lse_np = synth.kimi_lse(w)
        self.lse = torch.from_numpy(self.lse_np).to(dev)
        self.out = torch.empty((w.B, w.H, w.D), dtype=torch.float32, device=dev)
        self.glse = torch.empty((w.B, w.H), dtype=torch.float32, device=dev)
        torch.cuda.synchronize()
        print("# generated %s in %.1f s" % (w.describe(), time.time() - t0), file=sys.stderr, flush=True)
        self.bytes_call = algorithmic_bytes("kimi-rs", B)["combine"]

    def run(self, timing=None):
        from lse_weighted_merge_dcp_amd import sim

        sim.reduce_scatter_merge(self.part, self.lse, out=self.out, out_lse=self.glse, timing=timing)

    def kernels(self):
        return [("combine", self.bytes_call, [self.run])]

    def per_rank(self):
        """What one GPU of a real DCP group runs: rank 0's combine of its
        H/N-head slice of all N partials, as the exchange delivers it
        (received slices contiguous, [N, T, H/N, D]; the copy that stands in
        for the exchange is made once, untimed)."""
        import torch

        from lse_weighted_merge_dcp_amd import ops

        hs = self.w.H // self.w.N
        nbytes = algorithmic_bytes("kimi-rs", self.w.B)["combine_rank"]
        recv = self.part[:, :, :hs].contiguous()
        recv_lse = self.lse[:, :, :hs].contiguous()
        out = torch.empty((self.w.B, hs, self.w.D), dtype=torch.float32, device=self.dev)
        g = torch.empty((self.w.B, hs), dtype=torch.float32, device=self.dev)
        torch.cuda.synchronize()

        def call(timing=None):
            ops.dcp_lse_combine(recv, recv_lse, is_lse_base_on_e=True, out=out, out_lse=g, timing=timing)

        return [("combine", nbytes, [call])]

    def named_step(self):
        return [("combine", self.run)]

    def step_bytes(self):
        return self.bytes_call

    def config(self):
        w = self.w
        return {"workload": "Kimi-K3-shaped cached-extend merge, reduce-scatter flavour: N=8 ranks' partials "
                            "[%d, %d, %d] fp32, base-e LSE with 0.1%% NaN/inf, each rank's %d-head slice of the "
                            "output, no partial write-back" % (w.B, w.H, w.D, w.H // w.N),
                "N": w.N, "T": w.B, "H": w.H, "D": w.D, "payload_dtype": "f32"}

    def cpu_sample(self, budget_s):
        from oracle import oracle as orc

        w = self.w
        tblk = 64
        done, t_total = 0, 0.0
        while t_total < budget_s and done + tblk <= w.B:
            part = self.part[:, done:done + tblk].cpu().numpy()
            lse = self.lse_np[:, done:done + tblk]
            t0 = time.perf_counter()
            orc.combine(part, lse, "f32", False)
            t_total += time.perf_counter() - t0
            done += tblk
        per_tok = self.bytes_call / w.B
        return {"value": per_tok * done / t_total / 1e9, "unit": "GB/s", "cores": orc.num_threads(), "kind": "oracle",
                "sample": "first %d of %d tokens (all 8 ranks, 96 heads), %.1f s of CPU time, fp64" % (
                    done, w.B, t_total)}


# --------------------------------------------------------------------------
# timing
# --------------------------------------------------------------------------
def _median_event_s(fn, reps):
    import torch

    fn()
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        e1.synchronize()
        times.append(e0.elapsed_time(e1) * 1e-3)
    times.sort()
    return times[len(times) // 2]


def copy_ceiling_gbs(dev, nbytes=2 << 30, reps=10):
    """HBM rate of two plain copies of nbytes (read nbytes + write nbytes),
    timed with HIP events on the stream they run on: the runtime's
    device-to-device copy (torch copy_), and the library's own row copy (the
    N = 1 identity of dcp_unpack_combine: 1 KB rows copied bit for bit with
    16-byte vectors, the LSE word beside each row).  Returns
    {"runtime": GB/s, "library_row_copy": GB/s}."""
    import torch

    from lse_weighted_merge_dcp_amd import ops

    a = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    runtime = 2 * nbytes / _median_event_s(lambda: b.copy_(a), reps) / 1e9
    del b
    # the same bytes as [1, T, 1, 256] fp32 rows of 1 KB with one LSE each
    T = nbytes // 1024
    src = a.view(1, T, 1, 256)
    lse = torch.zeros((1, T, 1), dtype=torch.float32, device=dev)
    out = torch.empty((T, 1, 256), dtype=torch.float32, device=dev)
    g = torch.empty((T, 1), dtype=torch.float32, device=dev)
    moved = 2 * (nbytes + 4 * T)
    library = moved / _median_event_s(
        lambda: ops.dcp_lse_combine(src, lse, is_lse_base_on_e=True, out=out, out_lse=g), reps) / 1e9
    shape = launch_shape_of(lambda **kw: ops.dcp_lse_combine(src, lse, is_lse_base_on_e=True, out=out, out_lse=g,
                                                              **kw))
    del a, src, lse, out, g
    torch.cuda.empty_cache()
    return {"runtime": runtime, "library_row_copy": library, "library_row_copy_launch": [shape.blocks, shape.threads]}


def same_bytes_copy(dev, nbytes, reps):
    """The library's own row copy (the N = 1 identity of dcp_unpack_combine:
    1 KB rows plus their LSE words, copied bit for bit) moving about as many
    bytes as one launch of a kernel that moves nbytes, timed cold like the
    kernels: one launch per buffer set, as many sets as make at least 1 GiB
    of distinct source (at most 256), replayed in a HIP graph.  Returns
    {"bytes", "cold_us", "GBps", "sets"}: the rate a plain copy reaches at
    that size, fixed costs included."""
    import torch

    from lse_weighted_merge_dcp_amd import ops

    rows = max(1, int(round(nbytes / 2056)))        # each row: 1 KB + 4 B read, the same written
    moved = rows * 2056
    sets = max(1, min(256, math.ceil((1 << 30) / (rows * 1028))))
    bufs = []
    for _ in range(sets):
        src = torch.ones((1, rows, 1, 256), dtype=torch.float32, device=dev)
        lse = torch.zeros((1, rows, 1), dtype=torch.float32, device=dev)
        bufs.append((src, lse, torch.empty((rows, 1, 256), dtype=torch.float32, device=dev),
                     torch.empty((rows, 1), dtype=torch.float32, device=dev)))
    launches = [lambda b=b: ops.dcp_lse_combine(b[0], b[1], is_lse_base_on_e=True, out=b[2], out_lse=b[3])
                for b in bufs]
    us, _ = per_launch_us(launches, reps=reps)
    del launches, bufs
    torch.cuda.empty_cache()
    return {"bytes": moved, "cold_us": round(us, 3), "GBps": round(moved / (us * 1e-6) / 1e9, 1), "sets": sets}


def percentiles(xs):
    xs = sorted(xs)

    def q(f):
        return xs[min(len(xs) - 1, int(round(f * (len(xs) - 1))))]

    return {"p10": round(q(0.1), 4), "p50": round(q(0.5), 4), "p90": round(q(0.9), 4)}


def _graph_us(launches, reps, restore=None):
    import torch

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for f in launches:          # warm, outside the graph
            f()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in launches:
            f()
    torch.cuda.synchronize()
    total = 0.0
    stream = torch.cuda.current_stream()
    for _ in range(reps):
        if restore is not None:
            restore()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        g.replay()
        b.record(stream)
        b.synchronize()
        total += a.elapsed_time(b) * 1e3
    return total / (reps * len(launches)), g


def per_launch_us(launches, reps, restore=None, min_replay_us=1000.0):
    """Average duration of one launch: a HIP graph of the given launches is
    replayed `reps` times between two HIP events recorded on the stream the
    kernels run on.  A list whose replay is shorter than min_replay_us is
    repeated until it is not, so that the graph's own launch cost stays a
    small part of the figure.  Returns (us per launch, graph)."""
    us, g = _graph_us(launches, reps, restore)
    if us * len(launches) < min_replay_us:
        k = math.ceil(min_replay_us / max(us * len(launches), 1e-3))
        us, g = _graph_us(list(launches) * k, reps, restore)
    return us, g


def _sleep_cycles_per_ms():
    import torch

    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    torch.cuda._sleep(1_000_000)
    b.record()
    b.synchronize()
    return 1_000_000 / max(a.elapsed_time(b), 1e-3)


def in_step_us(named, reps, restore=None):
    """Average device time of each kernel inside the step.

    The step's calls are issued eagerly, in the step's order, behind a
    GPU-side wait (torch.cuda._sleep) that outlasts the host's enqueueing,
    so that the device runs them back to back as it runs the step graph.
    (A torch without _sleep runs the replays without that wait; the host
    may then fall behind the device, which leaves gaps between kernels but
    not inside the timed ones.)
    The launches of one kernel per replay carry timing events on their own
    dispatches (the timing= argument: the same kernels through the
    measurement library), so no marker packet sits between the kernels; the
    replays take the kernels in turn.  `named` is the step as
    (kernel name, call) pairs.  Returns ({name: us per launch}, {name:
    median device span in ms of the replays that timed it, from its first
    timed start to its last timed end})."""
    import torch

    from lse_weighted_merge_dcp_amd import timing

    order = []
    for n, _ in named:
        if n not in order:
            order.append(n)
    if restore:
        restore()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _, f in named:
        f()
    enqueue_ms = (time.perf_counter() - t0) * 1e3
    torch.cuda.synchronize()
    sleep = getattr(torch.cuda, "_sleep", None)
    gate = int(_sleep_cycles_per_ms() * (5.0 + 4.0 * enqueue_ms)) if sleep else 0
    events = [(timing.Event(), timing.Event()) for _ in named]
    total = {n: 0.0 for n in order}
    count = {n: 0 for n in order}
    spans = {n: [] for n in order}
    for r in range(reps * len(order)):
        name = order[r % len(order)]
        if restore:
            restore()
        if gate:
            sleep(gate)
        timed = [i for i, (n, _) in enumerate(named) if n == name]
        for i, (n, f) in enumerate(named):
            if n == name:
                f(timing=events[i])
            else:
                f()
        torch.cuda.synchronize()
        for i in timed:
            total[name] += events[i][0].elapsed_us(events[i][1])
            count[name] += 1
        spans[name].append(events[timed[0]][0].elapsed_us(events[timed[-1]][1]) / 1e3)
    return {n: total[n] / count[n] for n in order}, {n: round(percentiles(v)["p50"], 4) for n, v in spans.items()}


# The headline workload (the largest decode configuration: long-context
# decode, N = 16, B = 512) and the workloads reported beside it by default.
HEADLINE = ("longctx", None)
DEFAULT_SECONDARY = ("dsv3", "kimi")


def make_workload(key, B, layers, dev, kv=False):
    if key == "kimi":
        return InplaceWorkload(B, dev)
    if key == "kimi-rs":
        return ReduceScatterWorkload(B, dev)
    return A2AWorkload(key, B, layers, dev, kv=kv)


def time_step(wl, steps, warmup):
    """Capture the workload's step in one HIP graph, replay it `warmup`
    times, then time exactly `steps` replays bracketed by synchronisations
    (HIP events between replays give the per-step spread).  Returns (wall
    seconds of the timed region, [ms of each step])."""
    import torch

    restore = getattr(wl, "restore", None)
    step = [f for _, f in wl.named_step()]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(max(warmup, 1)):
            if restore:
                restore()
            for f in step:
                f()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for f in step:
            f()
    for _ in range(warmup):
        if restore:
            restore()
        graph.replay()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * steps)]
    if restore is None:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            ev[2 * i].record()
            graph.replay()
            ev[2 * i + 1].record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    else:
        # the in-place call destroys its input: restore it (untimed) before each step
        wall = 0.0
        for i in range(steps):
            restore()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            ev[2 * i].record()
            graph.replay()
            ev[2 * i + 1].record()
            torch.cuda.synchronize()
            wall += time.perf_counter() - t0
    del graph
    return wall, [ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(steps)]


def launch_shape_of(fn):
    """Launch shape of one call (launches, workgroups and threads of its
    last launch), from the measurement library."""
    import torch

    from lse_weighted_merge_dcp_amd import timing

    shape = timing.LaunchShape()
    fn(timing=(None, None, shape))
    torch.cuda.synchronize()
    return shape


def empty_floor_us(shape, count, reps):
    """Per-launch time of a graph of `count` launches of an empty kernel of
    the given launch shape: the fixed cost (dispatch, wave launch, drain) a
    launch of that shape pays whatever it does."""
    import torch

    from lse_weighted_merge_dcp_amd import timing

    def launch():
        timing.empty_kernel(shape.blocks, shape.threads, torch.cuda.current_stream().cuda_stream)

    us, _ = per_launch_us([launch] * count, reps=reps)
    return us


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def trace_lookup(key, kernel, shape, nbytes):
    """The committed rocprofv3 kernel-trace summaries' figures for the launches
    of this kernel at this launch shape (profiles/trace_*.json, the one named
    for this workload first), while the kernel sources still hash to what was
    traced; else None."""
    paths = sorted(glob.glob(os.path.join(ROOT, "profiles", "trace_*.json")))
    own = os.path.join(ROOT, "profiles", "trace_%s.json" % key)
    if own in paths:
        paths.remove(own)
        paths.insert(0, own)
    fam = {"pack": "pack_", "combine": "combine_", "inplace": "inplace_"}[kernel]
    src = kernel_source_hash()
    for p in paths:
        d = json.load(open(p))
        if d.get("kernel_source") != src:
            continue
        for e in d.get("launch_shapes", []):
            if e["kernel"].startswith(fam) and e["blocks"] == shape.blocks and e["threads"] == shape.threads:
                avg_us = e["avg_ns"] / 1e3
                return {"file": os.path.relpath(p, ROOT), "instance": e["kernel"], "launches": e["calls"],
                        "avg_us": round(avg_us, 3), "achieved": round(nbytes / (avg_us * 1e-6) / 1e9, 1),
                        "frac": round(nbytes / (avg_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                        "note": "rocprofv3 average over every launch of this kernel at this shape in the traced "
                                "bench.py command (in-step, cold and hot replays)"}
    return None


def measure(wl, key, B, args, full):
    """Every figure of one workload: the timed step, each kernel inside the
    step and cold, the cold layer, the roofline of the dominant kernel, the
    per-rank share against the empty-kernel floor, and (full) the
    cache-resident step, the copy ceiling and the CPU oracle."""
    import torch

    restore = getattr(wl, "restore", None)
    wall, step_ms = time_step(wl, args.steps, args.warmup)
    ms_per_step = wall / args.steps * 1e3
    gbs = wl.step_bytes() / (wall / args.steps) / 1e9
    layers = getattr(wl, "layers", 1)

    reps = max(3, args.steps // 4)
    in_step, spans = in_step_us(wl.named_step(), reps, restore=restore)
    kinfo = {}
    shapes = {}
    for name, nbytes, launches in wl.kernels():
        cold, _ = per_launch_us(launches, reps=reps, restore=restore)
        us = in_step[name]
        if restore:
            restore()
        shapes[name] = launch_shape_of(launches[0])
        kinfo[name] = {"us_per_launch": us, "bytes_per_launch": nbytes, "GBps": nbytes / (us * 1e-6) / 1e9,
                       "cold_us_per_launch": cold, "cold_GBps": nbytes / (cold * 1e-6) / 1e9,
                       "launch": [shapes[name].blocks, shapes[name].threads]}
        # a plain copy of the same size, cold: what the kernel's pattern
        # would reach if it were a copy, fixed costs of a launch that size
        # included
        kinfo[name]["copy_same_bytes"] = same_bytes_copy(wl.dev, nbytes, reps)
        kinfo[name]["of_copy_same_bytes"] = round(kinfo[name]["cold_GBps"] / kinfo[name]["copy_same_bytes"]["GBps"], 3)
    # every kernel of a layer run cold, one after the other: no layer's
    # inputs left in the caches by the kernel before it
    cold_us = sum(v["cold_us_per_launch"] for v in kinfo.values())
    layer_bytes = wl.step_bytes() // layers
    cold_layer = {"us": round(cold_us, 3), "GBps": round(layer_bytes / (cold_us * 1e-6) / 1e9, 1),
                  "pct_of_hbm_peak": round(100.0 * layer_bytes / (cold_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 2),
                  "note": "sum of each kernel's cold per-launch time (its launches back to back on distinct "
                          "buffers), free of data a previous kernel left in the Infinity Cache"}
    dom = max(kinfo, key=lambda k: kinfo[k]["us_per_launch"])
    achieved = kinfo[dom]["GBps"]
    ckey = counter_key(key, B)
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                "traffic": load_traffic(ckey, wl, dom),
                "timing": "inside the step: events on the kernel's own dispatches in eager replays of the step "
                          "(one kernel timed per replay)",
                "cold_achieved": round(kinfo[dom]["cold_GBps"], 1),
                "cold_frac": round(kinfo[dom]["cold_GBps"] / PEAK_HBM_GBS, 4),
                "trace": trace_lookup(ckey, dom, shapes[dom], kinfo[dom]["bytes_per_launch"])}
    res = {
        "value": round(gbs, 1),
        "pct_of_hbm_peak": round(100.0 * gbs / PEAK_HBM_GBS, 2),
        "ms_per_step": round(ms_per_step, 4),
        "us_per_layer": round(ms_per_step * 1e3 / layers, 3),
        "step_ms": percentiles(step_ms),
        "bytes_per_step": wl.step_bytes(),
        "kernels": {k: {kk: round(vv, 3) if isinstance(vv, float) else vv for kk, vv in v.items()}
                    for k, v in kinfo.items()},
        "cold_layer": cold_layer,
        "roofline": roofline,
        "timed_replay_span_ms": spans,
    }
    if hasattr(wl, "per_rank"):
        pr = {}
        for name, nbytes, launches in wl.per_rank():
            us, _ = per_launch_us(launches, reps=reps, restore=restore)
            if restore:
                restore()
            shp = launch_shape_of(launches[0])
            floor = empty_floor_us(shp, len(launches), reps)
            copy = same_bytes_copy(wl.dev, nbytes, reps)
            pr[name] = {"us_per_launch": round(us, 3), "bytes_per_launch": nbytes,
                        "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
                        "launch": [shp.blocks, shp.threads], "empty_kernel_us": round(floor, 3),
                        "net_GBps": round(nbytes / (max(us - floor, 1e-3) * 1e-6) / 1e9, 1),
                        "net_frac": round(nbytes / (max(us - floor, 1e-3) * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                        "copy_same_bytes": copy,
                        "of_copy_same_bytes": round(nbytes / (us * 1e-6) / 1e9 / copy["GBps"], 3)}
        if hasattr(wl, "hot_launches"):
            pr["us_per_layer"] = round(sum(v["us_per_launch"] for v in pr.values()), 3)
        pr["note"] = ("one rank's / one destination's own call at its real shape, cold; empty_kernel_us is a "
                      "graph of as many launches of an empty kernel with the same launch shape, net_GBps the "
                      "rate net of that fixed cost; copy_same_bytes the library's plain row copy of the same "
                      "size, cold, and of_copy_same_bytes the call's rate as a fraction of that copy's")
        res["per_rank"] = pr
    if full:
        if hasattr(wl, "hot_launches"):
            us, _ = per_launch_us(wl.hot_launches(), reps=reps)
            res["hot"] = {"us_per_layer": round(2 * us, 3),
                          "GBps": round(wl.bytes_layer / (2 * us * 1e-6) / 1e9, 1),
                          "note": "one layer's buffers reused by all layers (cache-resident)"}
        ceilings = copy_ceiling_gbs(wl.dev)
        res["copy_ceiling_launch"] = ceilings.pop("library_row_copy_launch")
        ceiling = max(ceilings.values())
        res["copy_ceiling_GBps"] = round(ceiling, 1)
        res["copy_ceilings_GBps"] = {k: round(v, 1) for k, v in ceilings.items()}
        res["pct_of_copy_ceiling"] = round(100.0 * gbs / ceiling, 2)
        if args.cpu_budget > 0:
            # the oracle on every host thread, then on one (a shorter sample)
            from oracle import oracle as orc

            cpu = wl.cpu_sample(args.cpu_budget)
            n_all = orc.num_threads()
            orc.set_num_threads(1)
            one = wl.cpu_sample(max(1.0, args.cpu_budget / 3))
            orc.set_num_threads(n_all)
            cpu["cpu_model"] = cpu_model()
            cpu["single_core"] = {"value": one["value"], "unit": one["unit"], "cores": one["cores"],
                                  "sample": one["sample"]}
            res["cpu_baseline"] = cpu
        else:
            res["cpu_baseline"] = None
    torch.cuda.synchronize()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None,
                    choices=["dsv3", "longctx", "split", "tiny", "kimi", "kimi-rs", "dsv3fp8"],
                    help="default: the long-context decode at B = 512, with dsv3 and kimi beside it")
    ap.add_argument("--B", type=int, default=None)
    ap.add_argument("--layers", type=int, default=61)
    ap.add_argument("--secondary", default=None,
                    help="comma-separated workloads measured after the headline and reported under "
                         "'secondary' (default: dsv3,kimi for the default run, none otherwise; 'none')")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of CPU oracle work (0 = skip)")
    ap.add_argument("--kv-len", action="store_true",
                    help="the pack reads per-rank KV lengths and neutralises tokens whose length is 0")
    ap.add_argument("--counter-run", action="store_true")
    ap.add_argument("--summarize-counters", default=None)
    ap.add_argument("--summarize-spread", default=None,
                    help="glob of counter-run logs of fresh processes -> profiles/spread_<key>.{json,md}")
    ap.add_argument("--summarize-trace", default=None,
                    help="rocprofv3 --kernel-trace --stats output directory -> profiles/trace_<key>.{json,md}")
    args = ap.parse_args()

    default_run = args.workload is None
    key = args.workload or HEADLINE[0]
    B = args.B if args.B is not None or not default_run else HEADLINE[1]
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, key, B)
        return
    if args.summarize_spread:
        summarize_spread(args.summarize_spread, key, B)
        return
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, key, B, command=os.environ.get("DCP_TRACE_COMMAND"),
                        bench_json=os.environ.get("DCP_TRACE_BENCH_JSON"))
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: it simulates all DCP ranks on a single MI355X "
              "(stacked in its HBM) and has no multi-GPU path; run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = make_workload(key, B, args.layers, dev, kv=args.kv_len)
    if args.counter_run:
        counter_run(wl)
        return

    head = measure(wl, key, B, args, full=True)
    config = wl.config()
    del wl
    torch.cuda.empty_cache()

    secondary = {}
    names = args.secondary
    if names is None:
        names = ",".join(DEFAULT_SECONDARY) if default_run else "none"
    for sk in [n for n in names.split(",") if n and n != "none"]:
        print("# secondary workload %s" % sk, file=sys.stderr, flush=True)
        w2 = make_workload(sk, None, args.layers, dev)
        r2 = measure(w2, sk, None, args, full=False)
        r2 = {"config": w2.config(), "unit": "GB/s", **r2}
        secondary[sk] = r2
        del w2
        torch.cuda.empty_cache()

    props = torch.cuda.get_device_properties(dev)
    device = {"arch": getattr(props, "gcnArchName", None), "compute_units": props.multi_processor_count,
              "memory_bytes": props.total_memory}
    res = {
        "metric": METRIC,
        "value": head.pop("value"),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head.pop("ms_per_step"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # the type the path computes in: LSE arithmetic and accumulation are fp32
        # for every payload type (the pack is a bit copy); the payload type
        # itself is config.payload_dtype
        "dtype": "f32",
        "data": "synthetic",
        "config": config,
        **head,
        "secondary": secondary,
        "kernel_source": kernel_source_hash(),
        "device": device,
    }
    print(json.dumps(res), flush=True)


def dpm_levels():
    """Current shader and memory clock levels from the amdgpu sysfs DPM
    tables (the entry marked '*'), for every card the process can see."""
    out = []
    for d in sorted(glob.glob("/sys/class/drm/card*/device")):
        for f in ("pp_dpm_sclk", "pp_dpm_mclk"):
            try:
                with open(os.path.join(d, f)) as fh:
                    cur = [ln.split(":", 1)[-1].replace("*", "").strip() for ln in fh if "*" in ln]
            except OSError:
                continue
            if cur:
                out.append("%s %s" % (f[len("pp_dpm_"):], cur[0]))
    return ", ".join(out) or "n/a"


def counter_run(wl):
    """For rocprofv3 --pmc: a plain elementwise pass over 1 GiB (the scale
    reference: 1 GiB read, 1 GiB written), then three calls of each kernel of
    the workload (its first three buffer sets, or its one call three times),
    each timed with events so that a counter pass also gives the rate of the
    allocation it ran on."""
    import torch

    n = 1 << 28
    a = torch.ones(n, dtype=torch.float32, device=wl.dev)
    b = torch.empty_like(a)
    for _ in range(3):
        torch.neg(a, out=b)   # one elementwise dispatch: reads 1 GiB, writes 1 GiB
    torch.cuda.synchronize()
    del a, b
    for name, nbytes, launches in wl.kernels():
        calls = (launches * 3)[:3]
        for i, f in enumerate(calls):
            if hasattr(wl, "restore"):
                wl.restore()
            # the counters serialise dispatches; events on the launching
            # stream still time this call alone
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            f()
            e1.record()
            e1.synchronize()
            us = e0.elapsed_time(e1) * 1e3
            print("# counter run: %s call %d: %.1f us, %.1f GB/s (clocks after it: %s)"
                  % (name, i, us, nbytes / us / 1e3, dpm_levels()), flush=True)
        print("# counter run: %s x%d, %d algorithmic bytes per launch" % (name, len(calls), nbytes), flush=True)


def counter_key(workload, B=None):
    """Name of a workload's counter summary (profiles/counters_<key>.json):
    the long-context sweep keeps one per batch size."""
    if workload == "longctx":
        from lse_weighted_merge_dcp_amd import synth

        return "longctx_B%d" % (B if B is not None else synth.WORKLOADS["longctx"].B)
    return workload


def load_traffic(key, wl, kernel):
    p = os.path.join(ROOT, "profiles", "counters_%s.json" % key)
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get("kernel_source") != kernel_source_hash() or kernel not in d.get("kernels", {}):
        return None
    return d["kernels"][kernel]["hbm_bytes_per_launch"]


def summarize_counters(directory, workload, B=None):
    """rocprofv3 --pmc CSVs (FETCH_SIZE run and WRITE_SIZE run) -> per-launch
    HBM bytes of each kernel, scaled by the copy reference."""
    import csv

    rows = []
    paths = []
    for d in directory.split(","):
        paths += glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    for path in paths:
        with open(path) as f:
            rows += list(csv.DictReader(f))
    by = {}
    for r in rows:
        name = r.get("Kernel_Name", "")
        cn = r.get("Counter_Name", "")
        val = float(r.get("Counter_Value", "nan"))
        by.setdefault((name, cn), []).append(val)

    def pick(pattern, cn):
        vals = [v for (k, c), vs in by.items() if re.search(pattern, k) and c == cn for v in vs]
        return sum(vals) / len(vals) if vals else None

    copy_bytes = 1 << 30      # torch.neg over 2^28 fp32: 1 GiB read, 1 GiB written
    f_copy = pick("neg_kernel", "FETCH_SIZE")
    w_copy = pick("neg_kernel", "WRITE_SIZE")
    if f_copy is None or w_copy is None:
        raise SystemExit("no copy-reference counters found in %s" % directory)
    fs = copy_bytes / f_copy       # bytes per counter unit, from a copy of known size
    ws = copy_bytes / w_copy
    key = counter_key(workload, B)
    out = {"kernel_source": kernel_source_hash(), "workload": workload, "key": key,
           "copy_reference": {"bytes": copy_bytes, "FETCH_SIZE": f_copy, "WRITE_SIZE": w_copy,
                              "fetch_scale": fs, "write_scale": ws}, "kernels": {}}
    for kname, pat in (("pack", r"\bpack_(stream_)?kernel"), ("combine", r"\bcombine_(wave_)?kernel"),
                       ("inplace", r"\binplace_kernel")):
        f = pick(pat, "FETCH_SIZE")
        wv = pick(pat, "WRITE_SIZE")
        if f is None or wv is None:
            continue
        out["kernels"][kname] = {"FETCH_SIZE": f, "WRITE_SIZE": wv, "read_bytes": f * fs, "write_bytes": wv * ws,
                                 "hbm_bytes_per_launch": f * fs + wv * ws}
    if workload == "longctx":
        out["B"] = int(key[len("longctx_B"):])
    alg = algorithmic_bytes(workload, out.get("B"))
    for kname, v in out["kernels"].items():
        v["algorithmic_bytes_per_launch"] = alg.get(kname)
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", "counters_%s.json" % key), "w") as fo:
        json.dump(out, fo, indent=1)
    with open(os.path.join(ROOT, "profiles", "counters_%s.md" % key), "w") as fo:
        fo.write(counters_markdown(out, directory))
    print(json.dumps(out, indent=1))


# counter sets of the placement study (one rocprofv3 --pmc pass each)
SPREAD_COUNTER_SETS = {
    "latency": "TCC_EA0_RDREQ_sum TCC_EA0_RDREQ_LEVEL_sum TCC_EA0_WRREQ_sum TCC_EA0_WRREQ_LEVEL_sum",
    "stalls": "TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum TCC_EA0_WRREQ_DRAM_CREDIT_STALL_sum TCC_TAG_STALL_sum "
              "GRBM_GUI_ACTIVE",
    "tlb": "TCP_UTCL1_TRANSLATION_MISS_sum TCP_UTCL1_TRANSLATION_HIT_sum "
           "TCP_UTCL1_STALL_UTCL2_REQ_OUT_OF_CREDITS_sum TCP_UTCL1_SERIALIZATION_STALL_sum",
}


def summarize_spread(pattern, workload, B=None, out_dir=None):
    """Runs of `bench.py --counter-run` in fresh processes (each its own
    allocation of the workload's buffers), plain or under one rocprofv3 --pmc
    pass -> profiles/spread_<key>.{json,md}.  PATTERN globs the runs' stdout
    logs; a counter pass keeps its rocprofv3 directory beside its log (the
    log's path without .log).  Per process: the rate of each call it timed,
    and per call of its kernel the counters of that pass (EA read and write
    latency from the in-flight levels, DRAM credit and tag stalls per busy
    cycle, L1 TLB misses)."""
    import csv
    import statistics

    key = counter_key(workload, B)
    fam = {"kimi": r"\binplace_kernel", "kimi-rs": r"\bcombine_(wave_)?kernel"}.get(workload, r"_kernel")
    procs = []
    for log in sorted(glob.glob(pattern)):
        text = open(log).read()
        rates = [float(m.group(1)) for m in re.finditer(r"# counter run: \S+ call \d+: [\d.]+ us, ([\d.]+) GB/s", text)]
        clocks = re.findall(r"# counter run: \S+ call \d+: .*\(clocks after it: ([^)]*)\)", text)
        if not rates:
            continue
        by = {}
        for path in glob.glob(os.path.join(log[:-len(".log")], "**", "*counter_collection.csv"), recursive=True):
            with open(path) as f:
                for r in csv.DictReader(f):
                    if re.search(fam, r.get("Kernel_Name", "")):
                        name = r["Counter_Name"][:-4] if r["Counter_Name"].endswith("_sum") else r["Counter_Name"]
                        by.setdefault(name, []).append(float(r["Counter_Value"]))
        m = {}
        if "TCC_EA0_RDREQ_LEVEL" in by:
            m["ea_read_latency_cycles"] = sum(by["TCC_EA0_RDREQ_LEVEL"]) / sum(by["TCC_EA0_RDREQ"])
        if "TCC_EA0_WRREQ_LEVEL" in by:
            m["ea_write_latency_cycles"] = sum(by["TCC_EA0_WRREQ_LEVEL"]) / sum(by["TCC_EA0_WRREQ"])
        if "GRBM_GUI_ACTIVE" in by:
            busy = sum(by["GRBM_GUI_ACTIVE"])
            for c, label in (("TCC_EA0_RDREQ_DRAM_CREDIT_STALL", "read_credit_stall_per_busy_cycle"),
                             ("TCC_EA0_WRREQ_DRAM_CREDIT_STALL", "write_credit_stall_per_busy_cycle"),
                             ("TCC_TAG_STALL", "tag_stall_per_busy_cycle")):
                if c in by:
                    m[label] = sum(by[c]) / busy
        if "TCP_UTCL1_TRANSLATION_MISS" in by:
            n = len(by["TCP_UTCL1_TRANSLATION_MISS"])
            m["utcl1_misses_per_call"] = sum(by["TCP_UTCL1_TRANSLATION_MISS"]) / n
            for c, label in (("TCP_UTCL1_STALL_UTCL2_REQ_OUT_OF_CREDITS", "utcl2_credit_stalls_per_call"),
                             ("TCP_UTCL1_SERIALIZATION_STALL", "utcl1_serialization_stalls_per_call")):
                if c in by:
                    m[label] = sum(by[c]) / n
        procs.append({"run": os.path.basename(log)[:-len(".log")], "counters": bool(by),
                      "rate_GBps": rates, "mean_GBps": sum(rates) / len(rates), "clocks": clocks, **m})
    if not procs:
        raise SystemExit("no counter-run logs match %s" % pattern)
    plain = [p["mean_GBps"] for p in procs if not p["counters"]]
    pmc = [p["mean_GBps"] for p in procs if p["counters"]]
    target = 0.7 * PEAK_HBM_GBS

    def stats(v):
        return {"processes": len(v), "median_GBps": statistics.median(v), "min_GBps": min(v), "max_GBps": max(v),
                "at_least_70pct": sum(x >= target for x in v)} if v else None

    out = {"kernel_source": kernel_source_hash(), "workload": workload, "key": key,
           "plain": stats(plain), "under_counters": stats(pmc), "processes": procs}
    out_dir = out_dir or os.path.join(ROOT, "profiles")
    os.makedirs(out_dir, exist_ok=True)
    with open(os.path.join(out_dir, "spread_%s.json" % key), "w") as fo:
        json.dump(out, fo, indent=1)
    with open(os.path.join(out_dir, "spread_%s.md" % key), "w") as fo:
        fo.write(spread_markdown(out, pattern))
    print(json.dumps({k: v for k, v in out.items() if k != "processes"}, indent=1))


def spread_markdown(d, pattern):
    w = d["workload"]
    cols = [("ea_read_latency_cycles", "EA read latency (cycles)", "%.0f"),
            ("ea_write_latency_cycles", "EA write latency (cycles)", "%.0f"),
            ("read_credit_stall_per_busy_cycle", "DRAM read credit stalls / busy cycle", "%.3f"),
            ("write_credit_stall_per_busy_cycle", "DRAM write credit stalls / busy cycle", "%.3f"),
            ("tag_stall_per_busy_cycle", "L2 tag stalls / busy cycle", "%.3f"),
            ("utcl1_misses_per_call", "L1 TLB misses per call", "%.0f"),
            ("utcl2_credit_stalls_per_call", "UTCL2 credit stalls per call", "%.0f")]

    def line(s, label):
        if not s:
            return "- %s: none" % label
        return ("- %s: %d processes, median %.0f GB/s (%.1f%% of 8 TB/s), range %.0f-%.0f GB/s, %d of them at "
                "70%% of peak or more" % (label, s["processes"], s["median_GBps"], s["median_GBps"] / PEAK_HBM_GBS * 100,
                                          s["min_GBps"], s["max_GBps"], s["at_least_70pct"]))

    lines = [
        "# Rate spread over allocations: %s workload" % w,
        "",
        "Kernel source hash `%s` (`spread_%s.json`).  Each row is a fresh process: it" % (d["kernel_source"], d["key"]),
        "allocates the workload's buffers, then times three calls of the kernel with",
        "events (`bench.py --counter-run`), either plain or under one rocprofv3 counter",
        "pass.  Commands (each run a new process, K numbering the runs):",
        "",
        "```",
        "cd /tmp && export TMPDIR=/tmp",
        "python3 $REPO/bench.py --workload %s --counter-run > $REPO/gpurun_out/ea_plainK.log" % w,
    ]
    for name, cs in SPREAD_COUNTER_SETS.items():
        lines.append("rocprofv3 --pmc %s --output-format csv -d $REPO/gpurun_out/ea_%sK -o run -- python3 "
                     "$REPO/bench.py --workload %s --counter-run > $REPO/gpurun_out/ea_%sK.log" % (cs, name, w, name))
    lines += [
        "python3 bench.py --workload %s --summarize-spread '%s'" % (w, pattern),
        "```",
        "",
        line(d["plain"], "plain"),
        line(d["under_counters"], "under a counter pass"),
        "",
        "| Run | GB/s (mean of its calls) | Calls | Clocks after its last call | "
        + " | ".join(c[1] for c in cols) + " |",
        "|---|---|---|---|" + "---|" * len(cols),
    ]
    for p in sorted(d["processes"], key=lambda p: (p["counters"], p["mean_GBps"])):
        cells = [(fmt % p[k]) if k in p else "" for k, _, fmt in cols]
        lines.append("| %s | %.0f | %s | %s | %s |" % (p["run"], p["mean_GBps"], ", ".join("%.0f" % r for r in p["rate_GBps"]),
                                                        (p.get("clocks") or ["n/a"])[-1], " | ".join(cells)))
    return "\n".join(lines) + "\n"


def counters_markdown(d, directory):
    w = d["workload"]
    key = d.get("key", w)
    wargs = w + (" --B %d" % d["B"] if "B" in d else "")
    dirs = directory.split(",")
    c = d["copy_reference"]
    lines = [
        "# HBM traffic counters: %s workload%s" % (w, " (B = %d)" % d["B"] if "B" in d else ""),
        "",
        "Kernel source hash `%s` (`counters_%s.json`; bench.py reports these bytes as" % (d["kernel_source"], key),
        "`roofline.traffic` only while the kernel sources still hash to it).  Two rocprofv3",
        "counter runs of the same short program (`bench.py --counter-run`: a 1 GiB",
        "`torch.neg` pass as the scale reference, then three launches of each kernel on",
        "the workload's buffers), then the summary:",
        "",
        "```",
        "cd /tmp && export TMPDIR=/tmp",
        "rocprofv3 --pmc FETCH_SIZE --output-format csv -d $REPO/%s -o run -- python3 $REPO/bench.py --workload %s --counter-run"
        % (dirs[0], wargs),
        "rocprofv3 --pmc WRITE_SIZE --output-format csv -d $REPO/%s -o run -- python3 $REPO/bench.py --workload %s --counter-run"
        % (dirs[-1], wargs),
        "python3 bench.py --workload %s --summarize-counters %s" % (wargs, directory),
        "```",
        "",
        "Scale reference: `torch.neg` over 2^28 fp32 reads and writes exactly 1 GiB; it",
        "reads FETCH_SIZE = %.0f and WRITE_SIZE = %.0f per dispatch, so one FETCH_SIZE" % (c["FETCH_SIZE"], c["WRITE_SIZE"]),
        "unit is %.0f bytes and one WRITE_SIZE unit %.0f bytes on this part." % (c["fetch_scale"], c["write_scale"]),
        "",
        "| Kernel | FETCH_SIZE | WRITE_SIZE | HBM read | HBM write | HBM total | Algorithmic | Ratio |",
        "|---|---|---|---|---|---|---|---|",
    ]
    for k, v in d["kernels"].items():
        a = v.get("algorithmic_bytes_per_launch")
        lines.append("| %s | %s | %s | %s | %s | %s | %s | %s |" % (
            k, "{:,.0f}".format(v["FETCH_SIZE"]), "{:,.0f}".format(v["WRITE_SIZE"]), _fmt_bytes(v["read_bytes"]),
            _fmt_bytes(v["write_bytes"]), _fmt_bytes(v["hbm_bytes_per_launch"]), _fmt_bytes(a) if a else "-",
            "%.3f" % (v["hbm_bytes_per_launch"] / a) if a else "-"))
    lines.append("")
    return "\n".join(lines)


def _short_kernel_name(name):
    """'void dcp::(anonymous namespace)::pack_stream_kernel<1, 8, true, false>(dcp::...)' ->
    'pack_stream_kernel<1, 8, true, false>'."""
    n = name.replace("(anonymous namespace)::", "").replace("dcp::", "")
    if n.startswith("void "):
        n = n[5:]
    depth = 0
    for i, ch in enumerate(n):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            return n[:i]
    return n


def _launch_roles(bench_json):
    """{(family, workgroups, threads): role} from the JSON line of the traced
    bench.py run (each kernel's and per-rank call's launch shape)."""
    roles = {}
    if not bench_json or not os.path.exists(bench_json):
        return roles
    with open(bench_json) as f:
        line = [ln for ln in f if ln.startswith("{")][-1]
    d = json.loads(line)

    def add(res, wname):
        for k, v in res.get("kernels", {}).items():
            if "launch" in v:
                roles.setdefault((k, v["launch"][0], v["launch"][1]), "%s, %s (every rank stacked)" % (wname, k))
        for k, v in (res.get("per_rank") or {}).items():
            if isinstance(v, dict) and "launch" in v:
                roles.setdefault((k, v["launch"][0], v["launch"][1]), "%s, one rank's %s" % (wname, k))

    add(d, d["config"]["workload"].split(":")[0])
    for name, sec in d.get("secondary", {}).items():
        add(sec, sec["config"]["workload"].split(":")[0])
    if "copy_ceiling_launch" in d:
        blocks, threads = d["copy_ceiling_launch"]
        roles.setdefault(("pack", blocks, threads), "the library's 2 GiB row copy (copy ceiling)")
    for (fam, blocks, threads), role in list(roles.items()):
        if "one rank's" in role:
            roles[("empty", blocks, threads)] = "empty kernel of the launch shape of " + role
    return roles


def summarize_trace(directory, workload, B=None, command=None, bench_json=None, out_dir=None):
    """rocprofv3 --kernel-trace --stats output (run_kernel_stats.csv and
    run_kernel_trace.csv under `directory`) -> profiles/trace_<key>.json and
    .md: every library kernel's launches grouped by instance and launch shape
    (workgroups x threads), with calls and average / min / max duration, and
    rocprofv3's own per-instance statistics.  bench.py reads the JSON back to
    set the traced average beside its own in-step figure."""
    import csv

    def find(suffix):
        hits = glob.glob(os.path.join(directory, "**", "*" + suffix), recursive=True)
        if not hits:
            raise SystemExit("no %s under %s" % (suffix, directory))
        return hits[0]

    stats = list(csv.DictReader(open(find("kernel_stats.csv"))))
    trace = list(csv.DictReader(open(find("kernel_trace.csv"))))
    groups = {}
    for r in trace:
        name = _short_kernel_name(r["Kernel_Name"])
        if not re.match(r"(pack_|combine_|inplace_|empty_kernel)", name):
            continue
        threads = int(r["Workgroup_Size_X"])
        blocks = int(r["Grid_Size_X"]) // max(threads, 1)
        dur = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        groups.setdefault((name, blocks, threads), []).append(dur)
    shapes = []
    for (name, blocks, threads), ds in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        shapes.append({"kernel": name, "blocks": blocks, "threads": threads, "calls": len(ds),
                       "avg_ns": sum(ds) / len(ds), "min_ns": min(ds), "max_ns": max(ds), "total_ns": sum(ds)})
    per_instance = []
    for r in stats:
        per_instance.append({"kernel": _short_kernel_name(r["Name"]), "calls": int(r["Calls"]),
                             "avg_ns": float(r["AverageNs"]), "min_ns": float(r["MinNs"]),
                             "max_ns": float(r["MaxNs"]), "percentage": float(r["Percentage"])})
    roles = _launch_roles(bench_json)
    for e in shapes:
        e["role"] = roles.get((e["kernel"].split("_")[0], e["blocks"], e["threads"]), "")
    key = counter_key(workload, B)
    out = {"kernel_source": kernel_source_hash(), "workload": workload, "key": key,
           "command": command, "launch_shapes": shapes, "stats": per_instance}
    out_dir = out_dir or os.path.join(ROOT, "profiles")
    os.makedirs(out_dir, exist_ok=True)
    with open(os.path.join(out_dir, "trace_%s.json" % key), "w") as fo:
        json.dump(out, fo, indent=1)
    lines = ["# Kernel trace: %s" % key, "",
             "Kernel source hash `%s` (`trace_%s.json`; bench.py reads it back for `roofline.trace`" % (
                 out["kernel_source"], key),
             "while the kernel sources still hash to it).", ""]
    if command:
        lines += ["Command:", "", "```", command, "```", ""]
    lines += ["rocprofv3 statistics (`kernel_stats.csv`, every launch of each instance, ns):", "",
              "| Kernel | Calls | Average ns | Min ns | Max ns | Share |", "|---|---|---|---|---|---|"]
    for e in per_instance:
        name = e["kernel"] if len(e["kernel"]) <= 100 else e["kernel"][:97] + "..."
        lines.append("| `%s` | %d | %s | %s | %s | %.1f%% |" % (
            name, e["calls"], "{:,.0f}".format(e["avg_ns"]), "{:,.0f}".format(e["min_ns"]),
            "{:,.0f}".format(e["max_ns"]), e["percentage"]))
    lines += ["", "The library's launches by launch shape (`kernel_trace.csv`; the role from the traced run's",
              "own JSON line, which records each call's launch shape):", "",
              "| Kernel | Workgroups x threads | Role | Calls | Average ns | Min ns | Max ns |",
              "|---|---|---|---|---|---|---|"]
    for e in shapes:
        lines.append("| `%s` | %d x %d | %s | %d | %s | %s | %s |" % (
            e["kernel"], e["blocks"], e["threads"], e["role"], e["calls"], "{:,.0f}".format(e["avg_ns"]),
            "{:,}".format(e["min_ns"]), "{:,}".format(e["max_ns"])))
    lines.append("")
    with open(os.path.join(out_dir, "trace_%s.md" % key), "w") as fo:
        fo.write("\n".join(lines))
    print(json.dumps({"key": key, "launch_shapes": shapes[:8]}, indent=1))


def _fmt_bytes(x):
    return "%.2f GB" % (x / 1e9) if x >= 1e9 else "%.2f MB" % (x / 1e6)


if __name__ == "__main__":
    main()
