"""The seeded input generators (CPU): determinism, the workloads' stated
laws, and the round-robin KV length model."""
import math

import numpy as np

from lse_weighted_merge_dcp_amd import synth
from oracle import attn_bruteforce as bf


def test_deterministic_and_seed_sensitive():
    w = synth.WORKLOADS["tiny"]
    a, b = synth.rank_inputs(w), synth.rank_inputs(w)
    assert np.array_equal(a["out"], b["out"]) and np.array_equal(a["lse"].view(np.uint32), b["lse"].view(np.uint32))
    c = synth.rank_inputs(synth.dataclasses.replace(w, seed=7))
    assert not np.array_equal(a["out"], c["out"])


def test_tiny_has_six_neutral_rows():
    inp = synth.rank_inputs(synth.WORKLOADS["tiny"])
    neutral = np.isneginf(inp["lse"])
    assert neutral.sum() == 6
    assert np.all(inp["out"][neutral] == 0)
    assert inp["out"].dtype == np.float32 and inp["out"].shape == (2, 4, 8, 64)


def test_dsv3_lse_follows_the_score_law():
    """lse = log2 sum 2^s over L ~ U{1024..16384} scores s ~ N(0,1): close to
    log2(L) + ln(2)/2 (the mean of 2^s is 2^(ln2/2))."""
    w = synth.WORKLOADS["dsv3"].with_batch(3)
    inp = synth.rank_inputs(w)
    L = inp["kv_len"]
    assert L.min() >= 1024 and L.max() <= 16384
    expect = np.log2(L)[..., None] + math.log(2) / 2
    sd = 1.1325 / np.sqrt(L)[..., None]          # spread of the sum, in log2 units
    assert np.all(np.abs(inp["lse"] - expect) < 6 * sd)
    assert abs(float(((inp["lse"] - expect) / sd).std()) - 1.0) < 0.1
    assert inp["out"].dtype == np.uint16 and inp["out"].shape == (8, 3, 128, 512)


def test_longctx_neutral_rows_and_law():
    w = synth.WORKLOADS["longctx"].with_batch(8)
    inp = synth.rank_inputs(w)
    L = inp["kv_len"]
    assert L[15, 0] == 0 and L.max() <= 65536
    empty = L == 0
    assert np.all(np.isneginf(inp["lse"][empty])) and np.all(inp["out"][empty] == 0)
    live = ~empty
    dev = inp["lse"][live] - (np.log2(L[live])[..., None] + math.log(2) / 2)
    assert np.abs(dev).max() < 6 * 1.1325 / math.sqrt(max(1, L[live].min()))


def test_kimi_lse_specials():
    w = synth.WORKLOADS["kimi"].with_batch(512)
    lse = synth.kimi_lse(w)
    total = lse.size
    k = int(round(0.001 * total))
    assert np.isnan(lse).sum() + np.isinf(lse).sum() == k
    assert abs(int(np.isnan(lse).sum()) - k / 3) <= 1 and abs(int(np.isposinf(lse).sum()) - k / 3) <= 1
    fin = lse[np.isfinite(lse)]
    assert abs(fin.mean() - 5.0) < 0.05 and abs(fin.std() - 4.0) < 0.05


def test_round_robin_lengths_partition_and_newest_owner():
    """Token t of a sequence belongs to rank t mod n: per-rank lengths sum to
    the global length, and appending one token grows exactly one rank, rank
    (L-1) mod n -- the two invariants of the sglang PR #33926 report's layout
    test (关键源码片段, TestDcpDecodeLayout), over the same sizes."""
    lens = np.arange(0, 41)
    for n in (1, 2, 3, 4, 8):
        total = sum(synth.dcp_local_len(lens, n, r) for r in range(n))
        np.testing.assert_array_equal(total, lens)
        for L in lens[1:]:
            grew = [int(synth.dcp_local_len(np.array([L]), n, r)[0] - synth.dcp_local_len(np.array([L - 1]), n, r)[0])
                    for r in range(n)]
            assert sum(grew) == 1 and grew[(L - 1) % n] == 1
        for L in (0, 7, 40):   # the same counts the brute-force split uses
            owner = bf.round_robin_owner(L, n)
            np.testing.assert_array_equal([int((owner == r).sum()) for r in range(n)],
                                          [int(synth.dcp_local_len(np.array([L]), n, r)[0]) for r in range(n)])
