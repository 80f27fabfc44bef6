"""CPU builds under AddressSanitizer and UndefinedBehaviorSanitizer (gcc, and
ROCm's clang for the HIP sources), with every report fatal (-fno-sanitize-recover=all):

* the fp64 oracle (oracle/dcp_oracle.c) built with both sanitizers, and the
  oracle pins and the two-oracle agreement tests run against that build in a
  child process (the sanitizer runtime preloaded, since Python itself is not
  instrumented);
* the host side of libdcpmerge's C ABI (csrc/api.cpp: argument validation,
  size limits and the element-to-byte stride conversion) driven by
  tests/host_validation_fuzz.cpp with extreme and random arguments, the
  kernel launchers replaced by recording stubs (no GPU, no HIP runtime);
* the real kernel launchers (pack.hip, combine.hip, inplace.hip compiled for
  the host only) behind the C ABI, driven by tests/host_launch_check.cpp
  with random valid calls, every launch checked against the grid limits;
* the fast division the kernels index with (csrc/fastdiv.hpp) and the
  XCD-aware workgroup orders (csrc/block_order.hpp).
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "lse_weighted_merge_dcp_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def runtime(name):
    path = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip("gcc has no %s here" % name)
    return path


def san_env(**extra):
    env = dict(os.environ)
    env["LD_PRELOAD"] = runtime("libasan.so") + ":" + runtime("libubsan.so")
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env.update(extra)
    return env


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    lib = str(tmp_path / "libdcp_oracle_san.so")
    subprocess.check_call(["gcc"] + SAN + ["-fopenmp", "-fno-fast-math", "-shared", "-fPIC", "-Wall", "-Wextra",
                                           os.path.join(ROOT, "oracle", "dcp_oracle.c"), "-o", lib, "-lm"])
    env = san_env(DCP_ORACLE_LIB=lib)
    # the child really loads the sanitizer build
    probe = subprocess.run([sys.executable, "-c", "from oracle import oracle as o; o.num_threads(); "
                            "print(any(%r in l for l in open('/proc/self/maps')))" % lib],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert probe.returncode == 0 and probe.stdout.strip() == "True", probe.stderr[-2000:]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        "tests/test_oracle_pins.py", "tests/test_oracle_twin.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert " passed" in r.stdout and "failed" not in r.stdout


def test_host_validation_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "host_validation_fuzz")
    subprocess.check_call(["g++", "-std=c++20", "-w", "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROCM, "include")]
                          + SAN + [os.path.join(ROOT, "tests", "host_validation_fuzz.cpp"),
                                   os.path.join(CSRC, "api.cpp"), "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    for seed in (1, 2, 3):
        r = subprocess.run([exe, "200000", str(seed)], capture_output=True, text=True, timeout=300, env=env)
        assert r.returncode == 0 and r.stdout.startswith("ok "), (r.stdout, r.stderr[-3000:])
        calls, accepted = map(int, r.stdout.split()[1:3])
        assert calls == 200000 and accepted > 1000


def test_fastdiv_under_asan_and_ubsan(tmp_path):
    from test_abi_host import FASTDIV_TEST

    src = tmp_path / "fd.cpp"
    src.write_text(FASTDIV_TEST)
    exe = str(tmp_path / "fd")
    subprocess.check_call(["g++", "-std=c++17", "-I" + CSRC] + SAN + [str(src), "-o", exe])
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.strip() == "0", (r.stdout, r.stderr[-2000:])


def test_block_orders_under_asan_and_ubsan(tmp_path):
    from test_abi_host import BLOCK_ORDER_TEST

    src = tmp_path / "bo.cpp"
    src.write_text(BLOCK_ORDER_TEST)
    exe = str(tmp_path / "bo")
    subprocess.check_call(["g++", "-std=c++17", "-I" + CSRC] + SAN + [str(src), "-o", exe])
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600,
                       env=dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1"))
    assert r.returncode == 0 and r.stdout.strip() == "0", (r.stdout, r.stderr[-2000:])


def _hipcc():
    cand = os.path.join(ROCM, "bin", "hipcc")
    if not os.path.exists(cand):
        pytest.skip("hipcc is not here")
    return cand


def _launch_check_exe(tmp_path, csrc, include, check_src, sanitize=True):
    """Build tests/host_launch_check.cpp against the host-only compile of the
    library sources in csrc (an empty device binary in place of the gfx950
    code; no HIP runtime linked: the check defines the entry points the
    launchers call)."""
    clangxx = os.path.join(ROCM, "lib", "llvm", "bin", "clang++")
    if not os.path.exists(clangxx):
        pytest.skip("ROCm's clang++ is not here")
    fatbin = tmp_path / "empty.fatbin"
    fatbin.write_bytes(b"")
    san = (["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=all",
            "-Xarch_host", "-fno-omit-frame-pointer"] if sanitize else [])
    host_only = [_hipcc(), "-x", "hip", "--cuda-host-only", "-std=c++20", "-O1", "-g", "-w", "-I" + include] + san + [
        "-Xclang", "-fcuda-include-gpubinary", "-Xclang", str(fatbin), "-c"]
    srcs = [os.path.join(csrc, f) for f in ("api.cpp", "bench_api.cpp", "pack.hip", "combine.hip", "inplace.hip")]
    srcs.append(check_src)
    objs = []
    for src in srcs:
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        subprocess.check_call(host_only + [src, "-o", obj])
        objs.append(obj)
    exe = str(tmp_path / "host_launch_check")
    subprocess.check_call([clangxx] + (["-fsanitize=address,undefined"] if sanitize else []) + ["-o", exe] + objs)
    return exe


def test_kernel_launches_under_asan_and_ubsan(tmp_path):
    """The real launchers of pack.hip, combine.hip and inplace.hip and the C
    ABIs of api.cpp and bench_api.cpp, compiled for the host only with ASan
    and UBSan, driven by tests/host_launch_check.cpp: random valid calls from
    tiny to far beyond one launch's reach, every launch checked against the
    grid limits, the timed calls' events and launch shapes against their
    contract."""
    exe = _launch_check_exe(tmp_path, CSRC, os.path.join(ROOT, "include"),
                            os.path.join(ROOT, "tests", "host_launch_check.cpp"))
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    for seed in (1, 2, 3):
        r = subprocess.run([exe, "20000", str(seed)], capture_output=True, text=True, timeout=300, env=env)
        assert r.returncode == 0 and r.stdout.startswith("ok "), (r.stdout, r.stderr[-3000:])
        calls, launches, most, items = map(int, r.stdout.split()[1:5])
        # every call launched, some needed several launches, and the largest grids reached the limit
        assert calls == 20000 and launches >= calls and most > 1 and items == 1 << 31


@pytest.mark.parametrize("path,old,new,message", [
    # launches allowed twice the workgroups: grids past 2^23 (2^32 work-items)
    ("dcp_launch.hpp", "kMaxBlocksPerLaunch = int64_t(1) << 23", "kMaxBlocksPerLaunch = int64_t(1) << 24",
     "launch outside the limits"),
    # the start event left on every launch of a call
    ("dcp_launch.hpp", "    t->start = nullptr;\n    return e;", "    return e;",
     "timing events or launch shape not as documented"),
])
def test_launch_check_rejects_planted_mistakes(tmp_path, path, old, new, message):
    """The launcher check has teeth: a copy of the library sources with one
    planted mistake (no sanitizers) must fail it with the matching report."""
    import shutil

    root = tmp_path / "src"
    csrc = root / "pkg" / "csrc"
    shutil.copytree(CSRC, csrc, ignore=shutil.ignore_patterns("_build", "__pycache__", "*.py"))
    shutil.copytree(os.path.join(ROOT, "include"), root / "include")
    (root / "tests").mkdir()
    text = (csrc / path).read_text()
    assert text.count(old) == 1, "the planted mistake no longer applies to %s" % path
    (csrc / path).write_text(text.replace(old, new))
    check = (root / "tests" / "host_launch_check.cpp")
    check.write_text(open(os.path.join(ROOT, "tests", "host_launch_check.cpp")).read().replace(
        '#include "../lse_weighted_merge_dcp_amd/csrc/dcpmerge_bench.h"', '#include "../pkg/csrc/dcpmerge_bench.h"'))
    exe = _launch_check_exe(tmp_path, str(csrc), str(root / "include"), str(check), sanitize=False)
    r = subprocess.run([exe, "20000", "1"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 1 and message in r.stderr, (r.returncode, r.stdout, r.stderr[-2000:])
