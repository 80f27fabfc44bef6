"""Planted mistakes in the oracle must fail at least one pin.

Each mutant is a one-line textual change to a copy of oracle/dcp_oracle.c
(a sign, a dropped term or guard, a wrong index, a wrong base), compiled to a
temporary library.  The pin suite below runs the same kinds of checks as
test_oracle_pins.py against that library; every mutant must fail it, and the
unmodified source must pass it.  Everything here runs on the CPU.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attn_bruteforce as bf
from oracle import oracle as orc

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(os.path.dirname(HERE), "oracle", "dcp_oracle.c")

MUTANTS = {
    "weight_sign": ("l[i * rows + r] - G", "G - l[i * rows + r]"),
    "no_guard_on_partial": ("double x = orc_guard(oi[d]);", "double x = oi[d];"),
    "no_guard_on_weight": ("double w = orc_guard(orc_pow_base(l[i * rows + r] - G, base2));",
                           "double w = orc_pow_base(l[i * rows + r] - G, base2);"),
    "no_inf_max_mask": ("if (isinf(m)) m = 0.0;", ""),
    "base_ignored": ("return base2 ? exp2(x) : exp(x);", "return exp(x);"),
    "log_base_ignored": ("return base2 ? log2(x) : log(x);", "return log(x);"),
    "peer_round_robin": ("int64_t p = h / Hpr;", "int64_t p = h % N;"),
    "local_head_wrong": ("int64_t hl = h % Hpr;", "int64_t hl = h / N;"),
    "first_peer_dropped": ("for (int64_t i = 0; i < N; ++i) {\n            double w",
                           "for (int64_t i = 1; i < N; ++i) {\n            double w"),
    "nan_lse_as_minus_inf": ("if (isnan(v)) return NAN;", "if (isnan(v)) return -INFINITY;"),
    "inplace_rank_index": ("l[(rank0 + j) * rows + r]", "l[j * rows + r]"),
    "no_single_rank_shortcut": ("        if (N == 1) {\n            g[r] = l[r];\n            for (int64_t d = 0; d < D; ++d) {\n                out[r * D + d] = o[r * D + d];",
                                "        if (N == 0) {\n            g[r] = l[r];\n            for (int64_t d = 0; d < D; ++d) {\n                out[r * D + d] = o[r * D + d];"),
    "lse_byte_swapped_peer": ("memcpy(dst_lse + p * dl_n + b * dl_b + hl * dl_h, src_lse",
                              "memcpy(dst_lse + hl * dl_n + b * dl_b + p * dl_h, src_lse"),
    "neutral_lse_sign": ("const float neg_inf = -INFINITY;", "const float neg_inf = INFINITY;"),
    "neutral_payload_kept": ("if (len == 0) {\n                for (int64_t d = 0; d < D; ++d)\n                    memset(",
                             "if (len == 0) {\n                for (int64_t d = 0; d < 0; ++d)\n                    memset("),
    "max_not_subtracted": ("s += orc_pow_base(l[i * stride] - m, base2);",
                           "s += orc_pow_base(l[i * stride], base2);"),
}


def _num(x):
    if isinstance(x, str):
        return {"nan": math.nan, "inf": math.inf, "-inf": -math.inf,
                "log2(3)": math.log2(3), "log2(5)": math.log2(5), "ln(2)": math.log(2)}[x]
    return float(x)


def _same(a, b, tol):
    if math.isnan(b):
        return math.isnan(a)
    if math.isinf(b):
        return a == b
    return abs(a - b) <= tol


def pin_suite(lib):
    """Return the list of pins that fail for this oracle library."""
    failed = []
    # hand-derived examples
    for c in json.load(open(os.path.join(HERE, "golden", "merge_cases.json")))["cases"]:
        lse = np.array([_num(x) for x in c["lse"]], np.float32)
        o = np.array([[_num(x) for x in row] for row in c["o"]], np.float32)
        N, D = o.shape
        out, g, _, _ = orc.combine(o.reshape(N, 1, 1, D), lse.reshape(N, 1, 1), "f32", c["base2"], lib=lib)
        ok = _same(g[0, 0], _num(c["G"]), 1e-12) and all(
            _same(a, _num(b), 1e-12) for a, b in zip(out[0, 0], c["out"]))
        if not ok:
            failed.append("golden:" + c["name"])
    # large LSE magnitudes against a library logsumexp (exercises the max shift)
    rng = np.random.default_rng(0)
    l = (rng.normal(0, 1, size=(4, 30)) + 800).astype(np.float32)
    o = rng.normal(size=(4, 30, 1, 2)).astype(np.float32)
    _, g, _, _ = orc.combine(o, l.reshape(4, 30, 1), "f32", False, lib=lib)
    ref = torch.logsumexp(torch.tensor(l.astype(np.float64)), 0).numpy()
    if not np.allclose(g[:, 0], ref, rtol=0, atol=1e-9):
        failed.append("library_logsumexp_large")
    # brute-force split attention, both bases
    for base2 in (False, True):
        q = rng.normal(size=(3, 8)); K = rng.normal(size=(21, 8)); V = rng.normal(size=(21, 5))
        outs, lses = bf.split_partials(q, K, V, 0.35, bf.round_robin_owner(21, 4), 4)
        fo, fl = bf.attention(q, K, V, 0.35)
        if base2:
            lses = lses * math.log2(math.e); fl = fl * math.log2(math.e)
        out, g, _, _ = orc.combine(outs.astype(np.float32).reshape(4, 1, 3, 5),
                                   lses.astype(np.float32).reshape(4, 1, 3), "f32", base2, lib=lib)
        if not (np.allclose(out[0], fo, atol=1e-5) and np.allclose(g[0], fl, atol=1e-5)):
            failed.append("bruteforce_base2=%s" % base2)
    # in-place: brute force through the held-rank subsets
    part = rng.normal(size=(4, 2, 3, 5)).astype(np.float32)
    lse4 = rng.normal(0, 2, size=(4, 2, 3)).astype(np.float32)
    _, full, gfull, _ = orc.inplace(part, lse4, "f32", False, lib=lib)
    want, gw, _, _ = orc.combine(part, lse4, "f32", False)      # the unmodified combine
    acc = np.zeros_like(full)
    for r0, P in ((0, 1), (1, 3)):
        _, o2, _, _ = orc.inplace(part[r0:r0 + P], lse4, "f32", False, rank0=r0, lib=lib)
        acc += o2
    if not (np.allclose(full, want, atol=1e-12) and np.allclose(acc, want, atol=1e-12)):
        failed.append("inplace_vs_combine")
    # pack: the page's view/permute construction
    N, B, Hpr, D = 4, 2, 3, 4
    H = N * Hpr
    out_t = torch.randn(B, H, D, generator=torch.Generator().manual_seed(1))
    lse_t = torch.randn(B, H, generator=torch.Generator().manual_seed(2))
    send = np.zeros((N, B, Hpr, D + 1), np.float32)
    orc.pack(out_t.numpy(), lse_t.numpy(), send[..., :D], send[..., D], N, lib=lib)
    if not (np.array_equal(send[..., :D], out_t.view(B, N, Hpr, D).permute(1, 0, 2, 3).numpy())
            and np.array_equal(send[..., D], lse_t.view(B, N, Hpr).permute(1, 0, 2).numpy())):
        failed.append("pack_page_construction")
    # pack with zero-KV tokens == pack of the explicitly neutralised inputs
    kv = np.array([3, 0], np.int32)
    o_n, l_n = out_t.numpy().copy(), lse_t.numpy().copy()
    o_n[1], l_n[1] = 0.0, -np.inf
    a = np.full((N, B, Hpr, D + 1), 5.0, np.float32)
    b_ = np.full((N, B, Hpr, D + 1), 5.0, np.float32)
    orc.pack(out_t.numpy(), lse_t.numpy(), a[..., :D], a[..., D], N, lib=lib, kv_len=kv)
    orc.pack(o_n, l_n, b_[..., :D], b_[..., D], N)
    if not np.array_equal(a.view(np.uint32), b_.view(np.uint32)):
        failed.append("pack_neutral_rows")
    return failed


def _build_variant(tmp_path, name, text):
    src = tmp_path / ("%s.c" % name)
    src.write_text(text)
    out = str(tmp_path / ("lib%s.so" % name))
    orc.compile_source(str(src), out)
    return orc.load_library(out)


def test_unmutated_oracle_passes_suite(tmp_path):
    lib = _build_variant(tmp_path, "orig", open(SRC).read())
    assert pin_suite(lib) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) >= 1, "mutation site not found: %s" % name
    lib = _build_variant(tmp_path, name, text.replace(old, new, 1))
    failed = pin_suite(lib)
    assert failed, "planted mistake %r passed every pin" % name


# --------------------------------------------------------------------------
# the fp8 (OCP E4M3) decoder of oracle/oracle.py: textual mutants of its
# source must fail its pin (torch's float8_e4m3fn over all 256 codes)
# --------------------------------------------------------------------------
FP8_MUTANTS = {
    "bias_8": ("2.0 ** (e - 7)", "2.0 ** (e - 8)"),
    "subnormal_scale": ("(m / 8.0) * 2.0 ** -6", "(m / 8.0) * 2.0 ** -7"),
    "ieee_top_exponent": ("if e == 0xF and m == 0x7:", "if e == 0xF:"),
    "sign_dropped": ("sign = -1.0 if c & 0x80 else 1.0", "sign = 1.0"),
    "no_implicit_one": ("(1.0 + m / 8.0)", "(m / 8.0)"),
    "four_mantissa_bits": ("e, m = (c >> 3) & 0xF, c & 0x7", "e, m = (c >> 4) & 0x7, c & 0xF"),
}


def _fp8_pin_holds(values) -> bool:
    codes = np.arange(256, dtype=np.uint8)
    got = values()
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    if not np.array_equal(np.isnan(got), np.isnan(want)):
        return False
    return bool(np.array_equal(got[~np.isnan(got)], want[~np.isnan(want)]))


def test_fp8_decoder_unmodified_passes_its_pin():
    assert _fp8_pin_holds(orc.fp8_e4m3_values)


@pytest.mark.parametrize("name", sorted(FP8_MUTANTS))
def test_fp8_decoder_mutant_fails_its_pin(name):
    import inspect
    import textwrap

    src = textwrap.dedent(inspect.getsource(orc.fp8_e4m3_values))
    old, new = FP8_MUTANTS[name]
    assert src.count(old) == 1, name
    ns = {"np": np, "math": math}
    exec(src.replace(old, new), ns)
    assert not _fp8_pin_holds(ns["fp8_e4m3_values"]), name
