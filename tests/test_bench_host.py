"""bench.py on the host (no GPU): the one-GPU guard and the algorithmic byte
counts behind every GB/s figure it prints."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")

import bench  # noqa: E402


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}), ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_exits_with_a_message(argv, env):
    e = dict(os.environ)
    e.update(env)
    r = subprocess.run([sys.executable, BENCH] + argv, capture_output=True, text=True, timeout=120, env=e)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_algorithmic_bytes_per_layer():
    """Per-layer bytes of the pack + combine path, (3N + 1)(D e + 4) per
    (token, head), and of the in-place and reduce-scatter merges."""
    b = bench.algorithmic_bytes("dsv3")
    assert b["pack"] + b["combine"] == 64 * 128 * (3 * 8 + 1) * (512 * 2 + 4) == 210_534_400
    assert b["pack"] == 134_742_016 and b["combine"] == 75_792_384
    for B, total in [(1, 6_447_616), (8, 51_580_928), (64, 412_647_424), (256, 1_650_589_696), (512, 3_301_179_392)]:
        b = bench.algorithmic_bytes("longctx", B)
        assert b["pack"] + b["combine"] == total == B * 128 * (3 * 16 + 1) * 1028
    assert bench.algorithmic_bytes("tiny")["pack"] + bench.algorithmic_bytes("tiny")["combine"] == 58_240
    split = bench.algorithmic_bytes("split")
    assert split["pack"] + split["combine"] == 256 * 64 * (3 * 4 + 1) * (128 * 2 + 4) == 55_377_920
    # in place: read N rows of 4D + 4, write N rows of 4D back and the merged row + G
    assert bench.algorithmic_bytes("kimi")["inplace"] == 16384 * 96 * 34_852 == 54_817_456_128
    # reduce-scatter flavour: no write-back
    assert bench.algorithmic_bytes("kimi-rs")["combine"] == 16384 * 96 * (8 * 2052 + 2052) == 29_047_652_352
    # one rank's own calls: scale its partial (read + write back, N LSEs), combine its 12-head slice
    assert bench.algorithmic_bytes("kimi")["inplace_rank"] == 16384 * 96 * (2 * 2048 + 8 * 4) == 6_492_782_592
    assert bench.algorithmic_bytes("kimi-rs")["combine_rank"] == 16384 * 12 * (8 * 2052 + 2052) == 3_630_956_544


def test_percentiles():
    p = bench.percentiles([5.0, 1.0, 3.0, 2.0, 4.0, 6.0, 7.0, 8.0, 9.0, 10.0, 11.0])
    assert p == {"p10": 2.0, "p50": 6.0, "p90": 10.0}


def test_fp8_bytes_and_counter_keys():
    """The fp8 decode layer: rows of D + 4 bytes (lpd = 4).  Counter
    summaries are kept per workload, and per batch size for the long-context
    sweep (its default batch is 512)."""
    b = bench.algorithmic_bytes("dsv3fp8")
    assert b["pack"] + b["combine"] == 64 * 128 * (3 * 8 + 1) * (512 + 4) == 105_676_800
    assert b["pack"] == 2 * 8 * 64 * 128 * 516 and b["combine"] == 9 * 64 * 128 * 516
    assert bench.counter_key("dsv3") == "dsv3" and bench.counter_key("kimi-rs") == "kimi-rs"
    assert bench.counter_key("longctx", 64) == "longctx_B64"
    assert bench.counter_key("longctx") == "longctx_B512"


def test_trace_summary_groups_launch_shapes_and_labels_them(tmp_path):
    """--summarize-trace: rocprofv3's kernel CSVs -> per (instance, launch
    shape) averages, labelled with the role the traced run's JSON line gives
    each launch shape; bench.py finds its dominant kernel's entry again."""
    import csv
    import json

    d = tmp_path / "prof"
    d.mkdir()
    pack = "void dcp::(anonymous namespace)::pack_stream_kernel<1, 8, true, false, true>(dcp::(anonymous namespace)::StreamK)"
    comb = "void dcp::(anonymous namespace)::combine_wave_kernel<dcp::BF16T, 16, true, 4, true>(dcp::(anonymous namespace)::CombK)"
    empty = "void (anonymous namespace)::empty_kernel()"
    rows = [(pack, 100, 460, 512, 147456), (pack, 500, 840, 512, 147456), (pack, 0, 30, 512, 9216),
            (comb, 1000, 1200, 256, 16384), (empty, 0, 5, 512, 9216),
            ("void at::cuda::(anonymous namespace)::spin_kernel(long)", 0, 99, 1, 1)]
    with open(d / "run_kernel_trace.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Workgroup_Size_X", "Grid_Size_X"])
        for name, t0, t1, wg, blocks in rows:
            w.writerow([name, t0, t1, wg, wg * blocks])
    with open(d / "run_kernel_stats.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "AverageNs", "MinNs", "MaxNs", "Percentage"])
        w.writerow([pack, 3, 263.3, 30, 360, 80.0])
    line = {"config": {"workload": "long-context decode sweep: N=16"},
            "kernels": {"pack": {"launch": [147456, 512]}, "combine": {"launch": [16384, 256]}},
            "per_rank": {"pack": {"launch": [9216, 512]}, "note": "x"}, "secondary": {}}
    bj = tmp_path / "bench.json"
    bj.write_text("# a log line\n" + json.dumps(line) + "\n")
    out = tmp_path / "out"
    bench.summarize_trace(str(d), "longctx", None, command="cmd", bench_json=str(bj), out_dir=str(out))
    t = json.load(open(out / "trace_longctx_B512.json"))
    by = {(e["kernel"], e["blocks"]): e for e in t["launch_shapes"]}
    p = by[("pack_stream_kernel<1, 8, true, false, true>", 147456)]
    assert p["calls"] == 2 and p["avg_ns"] == 350 and p["min_ns"] == 340 and p["max_ns"] == 360
    assert p["role"] == "long-context decode sweep, pack (every rank stacked)"
    assert by[("pack_stream_kernel<1, 8, true, false, true>", 9216)]["role"] == "long-context decode sweep, one rank's pack"
    assert by[("empty_kernel", 9216)]["role"].startswith("empty kernel of the launch shape of")
    assert by[("combine_wave_kernel<BF16T, 16, true, 4, true>", 16384)]["avg_ns"] == 200
    assert not any(e["kernel"].startswith("at::") for e in t["launch_shapes"])
    assert t["stats"][0]["kernel"] == "pack_stream_kernel<1, 8, true, false, true>"
    assert "| `pack_stream_kernel<1, 8, true, false, true>` | 147456 x 512 |" in (out / "trace_longctx_B512.md").read_text()
    assert bench._short_kernel_name("void at::cuda::(anonymous namespace)::spin_kernel(long)") == "at::cuda::spin_kernel"


def test_spread_summary_pairs_each_process_with_its_counters(tmp_path):
    """--summarize-spread: each fresh process's timed calls (from its
    counter-run log) with the counters of its kernel's launches (from the
    rocprofv3 directory beside the log); plain logs have no counters."""
    import csv
    import json

    kern = "void dcp::(anonymous namespace)::inplace_kernel<dcp::F32T, 16, 64, 8, 8, 1, true>(dcp::(anonymous namespace)::InplK)"

    def log(name, rates):
        (tmp_path / (name + ".log")).write_text("# generated\n" + "".join(
            "# counter run: inplace call %d: 10000.0 us, %.1f GB/s (clocks after it: sclk 2000Mhz, mclk 2000Mhz)\n"
            % (i, r) for i, r in enumerate(rates)) + "# counter run: inplace x3, 1 algorithmic bytes per launch\n")

    def counters(name, values):
        d = tmp_path / name
        d.mkdir()
        with open(d / "run_counter_collection.csv", "w", newline="") as f:
            w = csv.writer(f)
            w.writerow(["Kernel_Name", "Counter_Name", "Counter_Value"])
            for cn, vs in values.items():
                for v in vs:
                    w.writerow([kern, cn, v])
                    w.writerow(["void at::native::neg_kernel()", cn, 1.0])

    log("ea_plain1", [5400.0, 5500.0, 5600.0])
    log("ea_plain2", [6000.0, 6000.0, 6000.0])
    log("ea_latency1", [5700.0, 5700.0, 5700.0])
    counters("ea_latency1", {"TCC_EA0_RDREQ_sum": [100.0, 100.0], "TCC_EA0_RDREQ_LEVEL_sum": [300000.0, 340000.0],
                             "TCC_EA0_WRREQ_sum": [200.0, 200.0], "TCC_EA0_WRREQ_LEVEL_sum": [100000.0, 120000.0]})
    log("ea_tlb1", [5300.0, 5300.0, 5300.0])
    counters("ea_tlb1", {"TCP_UTCL1_TRANSLATION_MISS_sum": [65536.0, 65536.0],
                         "TCP_UTCL1_STALL_UTCL2_REQ_OUT_OF_CREDITS_sum": [0.0, 0.0]})
    out = tmp_path / "out"
    bench.summarize_spread(str(tmp_path / "ea_*.log"), "kimi", None, out_dir=str(out))
    d = json.load(open(out / "spread_kimi.json"))
    by = {p["run"]: p for p in d["processes"]}
    assert by["ea_plain1"]["mean_GBps"] == 5500.0 and not by["ea_plain1"]["counters"]
    assert by["ea_latency1"]["ea_read_latency_cycles"] == 3200.0
    assert by["ea_latency1"]["ea_write_latency_cycles"] == 550.0
    assert by["ea_tlb1"]["utcl1_misses_per_call"] == 65536.0
    assert by["ea_plain2"]["clocks"][-1] == "sclk 2000Mhz, mclk 2000Mhz"
    assert d["plain"] == {"processes": 2, "median_GBps": 5750.0, "min_GBps": 5500.0, "max_GBps": 6000.0,
                          "at_least_70pct": 1}
    assert d["under_counters"]["processes"] == 2 and d["under_counters"]["at_least_70pct"] == 1
    md = (out / "spread_kimi.md").read_text()
    assert "| ea_latency1 | 5700 | 5700, 5700, 5700 | sclk 2000Mhz, mclk 2000Mhz | 3200 | 550 |" in md
