"""GPU checks of the OCP FP8 E4M3 payload (e4m3fn) that hold exactly.

The merge of fp8 partials decodes each code to fp32, accumulates in fp32 and
rounds the result to nearest even in fp8.  Where the weights are exact (one
live peer: w = 1; two equal LSEs: w = 1/2) the fp32 sum is exact too, so the
output code is fixed bit for bit by the format alone.  The expected codes
come from torch's own float8_e4m3fn conversion on the CPU (round to nearest
even), independent of the library and of the oracle.  The other fp8 parity
tests (the workload, general shapes, special values, in-place) compare with
the fp64 oracle within half an fp8 ulp in test_gpu_pack/combine/inplace.
"""
import numpy as np
import pytest
import torch

from lse_weighted_merge_dcp_amd import ops

from helpers import say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
CODES = np.arange(256, dtype=np.uint8)


def values(codes: np.ndarray) -> np.ndarray:
    """fp64 value of fp8 codes, by torch's decoding."""
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def codes_of(x: np.ndarray) -> np.ndarray:
    """fp8 codes of fp64 values, by torch's conversion (round to nearest even)."""
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def merge(o_codes: np.ndarray, lse: np.ndarray, base_e: bool = True) -> np.ndarray:
    o = torch.from_numpy(np.ascontiguousarray(o_codes)).to(DEV).view(torch.float8_e4m3fn)
    out, _ = ops.dcp_lse_combine(o, torch.from_numpy(lse).to(DEV), is_lse_base_on_e=base_e)
    return out.cpu().view(torch.uint8).numpy()


@pytest.mark.parametrize("D", [256, 1024, 255])
def test_one_live_peer_returns_every_code(D):
    """Peer 1 neutral (LSE -inf), peer 0 live: w = (1, 0), so every finite
    code comes back unchanged (decode then encode are exact inverses; -0
    may come back as +0, the sign of zero is not compared) and the two NaN
    codes become 0 (nan_to_num).  D = 256: the short-row kernel; 1024: the
    row-per-wave kernel; 255: the element-granular kernel."""
    say("fp8 one live peer", D)
    B, Hpr = 3, 2
    rng = np.random.default_rng(D)
    o = rng.integers(0, 256, size=(2, B, Hpr, D), dtype=np.uint8)
    o[0].reshape(-1)[: (B * Hpr * D // 256) * 256] = np.tile(CODES, B * Hpr * D // 256)
    lse = np.zeros((2, B, Hpr), np.float32)
    lse[1] = -np.inf
    got = merge(o, lse)
    want = o[0].copy()
    nan = np.isnan(values(want))
    want[nan] = 0
    same = (got == want) | ((values(got) == 0) & (values(want) == 0))
    assert same.all(), "%d codes differ, first %s" % (int((~same).sum()), np.argwhere(~same)[:4].tolist())


@pytest.mark.parametrize("base_e", [True, False])
def test_two_equal_peers_round_to_nearest_even(base_e):
    """Equal LSEs give w = 1/2 exactly, so out = RNE((a + b) / 2) for every
    pair of codes (a, b): 65,536 pairs, about half of them exact ties between
    two fp8 neighbours, each checked against torch's conversion.  NaN
    operands count as 0."""
    say("fp8 pairs", base_e)
    o = np.empty((2, 256, 1, 256), np.uint8)
    o[0] = CODES[:, None, None]          # a = row code
    o[1] = CODES[None, None, :]          # b = column code
    lse = np.full((2, 256, 1), 1.5, np.float32)
    got = merge(o, lse, base_e)
    a = np.nan_to_num(values(o[0]), nan=0.0)
    b = np.nan_to_num(values(o[1]), nan=0.0)
    want = codes_of((a + b) / 2)
    same = (got == want) | ((values(got) == 0) & (values(want) == 0))   # the sign of zero is not compared
    assert same.all(), "%d of 65536 pairs differ, first %s" % (int((~same).sum()), np.argwhere(~same)[:4].tolist())


@pytest.mark.parametrize("sign", [1.0, -1.0])
def test_largest_value_merges_to_itself(sign):
    """Eight peers all holding +-448 (the largest finite fp8 value) with
    random LSEs: the weights sum to 1 within fp32 rounding, and the merged
    value must come back as +-448, never as NaN or a smaller code."""
    say("fp8 largest", sign)
    N, B, Hpr, D = 8, 16, 4, 512
    o = np.full((N, B, Hpr, D), codes_of(np.array([sign * 448.0]))[0], np.uint8)
    lse = np.random.default_rng(7).normal(0, 2, size=(N, B, Hpr)).astype(np.float32)
    got = merge(o, lse)
    assert np.array_equal(values(got), np.full(got.shape, sign * 448.0))


def test_encoder_is_nearest_even_on_every_fp32_pattern():
    """tests/fp8_encode_check.hip: the kernels' fp8 encoder (gfx950's packed
    conversion behind a saturation at 448) against a table-based
    nearest-even reference written from the format's definition, on all
    2^32 fp32 bit patterns in both halves of the packed word; NaN must give
    a NaN code."""
    import os
    import subprocess

    exe = os.path.join(os.path.dirname(os.path.abspath(__file__)), "fp8_encode_check")
    assert os.path.exists(exe), "tests/fp8_encode_check is not built: run __graft_entry__.build()"
    say("fp8 encode check over every fp32 pattern")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, (r.stdout, r.stderr)
    assert "total 4294967296 patterns, 0 differ" in r.stdout, r.stdout
