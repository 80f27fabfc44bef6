"""Seeded synthetic inputs for the DCP partial-merge path.

This module serves both the HIP path and the oracle: it only draws random
numbers and shapes them like the pages' workloads.  It holds none of the
merge's arithmetic (no global LSE, no weights, no weighted sum).

Workloads (the pages measure on DeepSeek-V3.x MLA decode and on Kimi-K3
cached extend; no dataset or weights are involved, so these seeded draws
stand in for them):

  1 "tiny"      N=2 ranks, B=4 tokens, H=8 heads, D=64, fp32, base-e LSE.
                out ~ N(0,1), lse ~ N(0,3); 6 of the 64 (rank, token, head)
                rows are neutral (out = 0, lse = -inf).
  2 "dsv3"      N=8, B=64, H=128 (16 per rank), D=512 (kv_lora_rank), bf16,
                base-2 LSE.  Per (rank, token) a KV length L ~ U{1024..16384};
                lse[r,b,h] = log2 of the sum of 2^s over L scores s ~ N(0,1)
                (the attention kernel's own LSE of synthetic scores: fp32 exp2
                of each score, summed in fp64).
  3 "split"     N=4, B=256, H=64 (16 per rank), D=128, fp16, base-e LSE ~ N(0,3).
  4 "kimi"      N=8 ranks' partials [T=16384, H=96, D=512] fp32, base-e
                LSE ~ N(5,4); 0.1% of the LSE entries are NaN, +inf or -inf
                (equal thirds) at seeded positions.
  5 "longctx"   N=16, H=128 (8 per rank), D=512, bf16, base-2 LSE, B in
                {1, 8, 64, 256, 512}.  L[r,b] ~ U{0..65536} and L[15,0] = 0.
                L = 0 gives a neutral row; otherwise out ~ N(0,1) and
                lse = log2(L) + ln(2)/2 + 1.1325 z / sqrt(L), z ~ N(0,1): the
                large-L distribution of log2 sum 2^s for L scores s ~ N(0,1)
                (mean of 2^s is 2^(ln2/2); the relative spread of the sum is
                sqrt(e^(ln2^2) - 1)/sqrt(L) = 0.785/sqrt(L), i.e. 1.1325/sqrt(L)
                in log2 units), drawn directly because exact draws would take
                3.4e10 samples at B = 512.
  6 "dsv3fp8"   the shape of 2 with an OCP FP8 E4M3 payload (out ~ N(0,1)
                rounded to fp8), base-2 LSE from the law of 5 over
                L ~ U{1024..16384}.

N(a, b) means mean a, standard deviation b.  Every draw comes from a
generator seeded by (seed, workload, rank, stream), so any rank's data can be
regenerated on its own and the result does not depend on thread counts.

Payload arrays are numpy arrays in the storage type: float32, float16,
uint16 holding bf16 bits, or uint8 holding fp8 codes (bf16 and fp8 values
are float32 draws rounded to nearest even by torch's conversion).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

ESIZE = {"f32": 4, "f16": 2, "bf16": 2, "fp8": 1}
# numpy storage of each payload type: bf16 as raw uint16 bits, fp8 (OCP E4M3)
# as raw uint8 codes
NP_STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16, "fp8": np.uint8}
LONGCTX_BATCHES = (1, 8, 64, 256, 512)


@dataclasses.dataclass(frozen=True)
class Workload:
    key: str
    index: int
    N: int
    B: int          # tokens (T for the in-place workload)
    H: int
    D: int
    dtype: str      # "f32" | "f16" | "bf16" | "fp8"
    base2: bool
    layout: str     # "interleaved" | "split" | "inplace"
    seed: int

    @property
    def Hpr(self) -> int:
        return self.H // self.N

    @property
    def esize(self) -> int:
        return ESIZE[self.dtype]

    def with_batch(self, B: int) -> "Workload":
        return dataclasses.replace(self, B=B)

    def describe(self) -> str:
        return "%s: N=%d B=%d H=%d D=%d %s base-%s %s" % (
            self.key, self.N, self.B, self.H, self.D, self.dtype, "2" if self.base2 else "e", self.layout)


WORKLOADS = {
    "tiny": Workload("tiny", 1, N=2, B=4, H=8, D=64, dtype="f32", base2=False, layout="interleaved", seed=0),
    "dsv3": Workload("dsv3", 2, N=8, B=64, H=128, D=512, dtype="bf16", base2=True, layout="interleaved", seed=1),
    "split": Workload("split", 3, N=4, B=256, H=64, D=128, dtype="f16", base2=False, layout="split", seed=2),
    "kimi": Workload("kimi", 4, N=8, B=16384, H=96, D=512, dtype="f32", base2=False, layout="inplace", seed=3),
    "longctx": Workload("longctx", 5, N=16, B=512, H=128, D=512, dtype="bf16", base2=True,
                        layout="interleaved", seed=4),
    "dsv3fp8": Workload("dsv3fp8", 6, N=8, B=64, H=128, D=512, dtype="fp8", base2=True, layout="interleaved",
                        seed=5),
}


# --------------------------------------------------------------------------
# seeded generators
# --------------------------------------------------------------------------
def np_rng(w: Workload, rank: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, w.index, rank, stream])))


def torch_gen(w: Workload, rank: int, stream: int) -> torch.Generator:
    s = np.random.SeedSequence([w.seed, w.index, rank, stream, 7]).generate_state(1, np.uint64)[0]
    return torch.Generator().manual_seed(int(s & 0x7FFFFFFFFFFFFFFF))


def to_storage(x: torch.Tensor, dtype: str) -> np.ndarray:
    """float32 CPU tensor -> numpy storage array of the payload type (RNE)."""
    if dtype == "f32":
        return x.numpy()
    if dtype == "f16":
        return x.to(torch.float16).numpy()
    if dtype == "bf16":
        return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    if dtype == "fp8":
        return x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    raise ValueError(dtype)


def _normal_rows(w: Workload, rank: int, shape, stream: int = 0) -> np.ndarray:
    return to_storage(torch.randn(*shape, generator=torch_gen(w, rank, stream)), w.dtype)


def rank_inputs(w: Workload):
    """All N ranks' rank-local partials.

    Returns dict(out=[N,B,H,D] storage array, lse=[N,B,H] float32,
    kv_len=[N,B] int64 or None).
    """
    N, B, H, D = w.N, w.B, w.H, w.D
    out = np.empty((N, B, H, D), NP_STORAGE[w.dtype])
    lse = np.empty((N, B, H), np.float32)
    kv_len = None
    if w.key == "tiny":
        for r in range(N):
            out[r] = _normal_rows(w, r, (B, H, D))
            lse[r] = np_rng(w, r, 1).normal(0.0, 3.0, size=(B, H))
        k = int(round(0.1 * N * B * H))
        pick = np_rng(w, N, 2).choice(N * B * H, size=k, replace=False)
        flat_o = out.reshape(N * B * H, D)
        flat_l = lse.reshape(-1)
        flat_o[pick] = 0
        flat_l[pick] = -np.inf
    elif w.key == "dsv3":
        kv_len = np.empty((N, B), np.int64)
        for r in range(N):
            out[r] = _normal_rows(w, r, (B, H, D))
            kv_len[r] = np_rng(w, r, 1).integers(1024, 16384, size=B, endpoint=True)
            g = torch_gen(w, r, 2)
            for b in range(B):
                s = torch.randn(H, int(kv_len[r, b]), generator=g)
                lse[r, b] = torch.log2(torch.exp2(s).sum(dim=1, dtype=torch.float64)).to(torch.float32).numpy()
    elif w.key == "dsv3fp8":
        # the DeepSeek-V3 shape with an fp8 payload; LSEs from the large-L law
        # of the long-context recipe over L ~ U{1024..16384}
        kv_len = np.empty((N, B), np.int64)
        for r in range(N):
            out[r] = _normal_rows(w, r, (B, H, D))
            kv_len[r] = np_rng(w, r, 1).integers(1024, 16384, size=B, endpoint=True)
            z = np_rng(w, r, 2).normal(0.0, 1.0, size=(B, H))
            L = kv_len[r].astype(np.float64)[:, None]
            lse[r] = np.log2(L) + math.log(2.0) / 2.0 + 1.1325 * z / np.sqrt(L)
    elif w.key == "split":
        for r in range(N):
            out[r] = _normal_rows(w, r, (B, H, D))
            lse[r] = np_rng(w, r, 1).normal(0.0, 3.0, size=(B, H))
    elif w.key == "kimi":
        for r in range(N):
            out[r] = _normal_rows(w, r, (B, H, D))
        lse[:] = kimi_lse(w)
    elif w.key == "longctx":
        kv_len = longctx_lengths(w)
        for r in range(N):
            out[r] = _normal_rows(w, r, (B, H, D))
            z = np_rng(w, r, 1).normal(0.0, 1.0, size=(B, H))
            L = np.maximum(kv_len[r], 1).astype(np.float64)[:, None]
            lse[r] = np.log2(L) + math.log(2.0) / 2.0 + 1.1325 * z / np.sqrt(L)
            empty = kv_len[r] == 0
            out[r][empty] = 0
            lse[r][empty] = -np.inf
    else:
        raise KeyError(w.key)
    return {"out": out, "lse": lse, "kv_len": kv_len}


def longctx_lengths(w: Workload) -> np.ndarray:
    """Per (rank, token) KV lengths of the long-context workload; L[N-1, 0] = 0."""
    L = np.stack([np_rng(w, r, 3).integers(0, 65536, size=w.B, endpoint=True) for r in range(w.N)])
    L[w.N - 1, 0] = 0
    return L.astype(np.int64)


def kimi_lse(w: Workload) -> np.ndarray:
    """[N,T,H] float32 base-e LSE ~ N(5,4) with 0.1% NaN/+inf/-inf at seeded positions."""
    N, T, H = w.N, w.B, w.H
    lse = np.empty((N, T, H), np.float32)
    for r in range(N):
        lse[r] = np_rng(w, r, 1).normal(5.0, 4.0, size=(T, H))
    total = N * T * H
    k = int(round(0.001 * total))
    pick = np_rng(w, N, 2).choice(total, size=k, replace=False)
    flat = lse.reshape(-1)
    thirds = np.array_split(pick, 3)
    flat[thirds[0]] = np.nan
    flat[thirds[1]] = np.inf
    flat[thirds[2]] = -np.inf
    return lse


# tokens per seeded draw of the in-place workload's device partials
KIMI_TOKEN_BLOCK = 2048


def _kimi_block_generator(w: Workload, rank: int, t0: int, device) -> torch.Generator:
    s = np.random.SeedSequence([w.seed, w.index, rank, 4, t0]).generate_state(1, np.uint64)[0]
    return torch.Generator(device=device).manual_seed(int(s & 0x7FFFFFFFFFFFFFFF))


def kimi_partial_device(w: Workload, device, dtype=torch.float32) -> torch.Tensor:
    """The in-place workload's partial stack [N,T,H,D] drawn directly in device
    memory (24 GiB at the full size): N(0,1) from a device generator seeded per
    (rank, block of KIMI_TOKEN_BLOCK tokens).  Deterministic for a given seed
    on a given device type."""
    N, T, H, D = w.N, w.B, w.H, w.D
    part = torch.empty((N, T, H, D), dtype=dtype, device=device)
    for r in range(N):
        for t0 in range(0, T, KIMI_TOKEN_BLOCK):
            t1 = min(T, t0 + KIMI_TOKEN_BLOCK)
            part[r, t0:t1].normal_(0.0, 1.0, generator=_kimi_block_generator(w, r, t0, device))
    return part


def kimi_partial_block_device(w: Workload, device, t0: int, dtype=torch.float32) -> torch.Tensor:
    """Tokens [t0, t0 + KIMI_TOKEN_BLOCK) of kimi_partial_device's stack,
    [N, tokens, H, D], drawn again from the same seeds (t0 must start a
    block): the pristine partials of that block, for checking a merge that
    overwrote them."""
    assert t0 % KIMI_TOKEN_BLOCK == 0 and 0 <= t0 < w.B
    t1 = min(w.B, t0 + KIMI_TOKEN_BLOCK)
    blk = torch.empty((w.N, t1 - t0, w.H, w.D), dtype=dtype, device=device)
    for r in range(w.N):
        blk[r].normal_(0.0, 1.0, generator=_kimi_block_generator(w, r, t0, device))
    return blk


def dcp_local_len(L: np.ndarray, n: int, rank: int) -> np.ndarray:
    """Round-robin KV ownership (sglang PR #33926 report, 关键源码片段): token t
    of a length-L sequence belongs to rank t mod n, so rank `rank` owns
    L // n tokens plus one more when rank < L mod n."""
    L = np.asarray(L)
    return L // n + (rank < (L % n)).astype(L.dtype)
