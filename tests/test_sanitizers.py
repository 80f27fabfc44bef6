"""CPU builds under AddressSanitizer and UndefinedBehaviorSanitizer (gcc),
with every report fatal (-fno-sanitize-recover=all):

* the fp64 oracle (oracle/dcp_oracle.c) built with both sanitizers, and the
  oracle pins and the two-oracle agreement tests run against that build in a
  child process (the sanitizer runtime preloaded, since Python itself is not
  instrumented);
* the host side of libdcpmerge's C ABI (csrc/api.cpp: argument validation,
  size limits and the element-to-byte stride conversion) driven by
  tests/host_validation_fuzz.cpp with extreme and random arguments, the
  kernel launchers replaced by recording stubs (no GPU, no HIP runtime);
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
