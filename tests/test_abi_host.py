"""Host-side checks of the C ABI (no GPU, no kernel launch).

* the shared library loads and exports every function include/dcpmerge.h
  declares, and nothing else; the measurement library libdcpmerge_bench.so
  exports exactly the timed calls its own header declares;
* dcp_lse_pack_dim and dcp_status_str;
* every validation error is returned before anything is enqueued (the calls
  below use fake, never-dereferenced addresses; only rejected or zero-sized
  calls are made, so no kernel is launched);
* the fast-division helper the kernels index with, compiled for the host.
"""
import ctypes
import os
import re
import subprocess

import pytest
import torch

from lse_weighted_merge_dcp_amd import _lib, ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dcpmerge.h")
CSRC = os.path.join(ROOT, "lse_weighted_merge_dcp_amd", "csrc")

OK, NULL, SHAPE, HEADS, DTYPE, BASE, STRIDE, ALIGN, HRANGE = 0, -1, -2, -3, -4, -5, -6, -7, -8
A = 0x100000  # fake 256-aligned address, never dereferenced


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(dcp_\w+)\s*\(", text, re.M)))


BENCH_HEADER = os.path.join(CSRC, "dcpmerge_bench.h")


def declared_in(path, prefix):
    text = open(path).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(%s\w+)\s*\(" % prefix, text, re.M)))


def exported_functions(path):
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True, check=True)
    return sorted(set(re.findall(r" T (\w+)$", out.stdout, re.M)))


def test_header_declares_the_entry_points():
    assert declared_functions() == ["dcp_lse_combine_inplace", "dcp_lse_pack_dim", "dcp_pack",
                                    "dcp_status_str", "dcp_unpack_combine"]


def test_library_exports_exactly_the_declared_symbols():
    """libdcpmerge.so exports the calls of include/dcpmerge.h and nothing
    else (no timing hook, no internal C++ symbol)."""
    lib = _lib.lib()
    assert exported_functions(_lib.LIB_PATH) == declared_functions()
    for name in declared_functions():
        assert getattr(lib, name) is not None
        assert name in _lib.SIGNATURES


def test_bench_library_exports_exactly_its_timed_calls():
    """libdcpmerge_bench.so exports the dcpb_* calls of its header, one per
    compute call of libdcpmerge, each with two event arguments in front."""
    from lse_weighted_merge_dcp_amd import timing

    declared = declared_in(BENCH_HEADER, "dcpb_")
    assert declared == ["dcpb_empty_kernel", "dcpb_lse_combine_inplace", "dcpb_pack", "dcpb_unpack_combine"]
    assert exported_functions(timing.BENCH_LIB_PATH) == declared
    lib = timing.bench_lib()
    for name in declared[1:]:
        assert len(getattr(lib, name).argtypes) == len(_lib.SIGNATURES["dcp_" + name[5:]][0]) + 3
    assert lib.dcpb_empty_kernel(0, 64, None) == SHAPE and lib.dcpb_empty_kernel(1, 2048, None) == SHAPE


def test_timing_module_names():
    """Every name the timing module uses at run time is defined (its GPU
    paths only run on the GPU machine)."""
    import ast
    import builtins

    from lse_weighted_merge_dcp_amd import timing

    tree = ast.parse(open(timing.__file__).read())
    defined = set(dir(timing)) | set(dir(builtins))
    for node in ast.walk(tree):
        if isinstance(node, (ast.FunctionDef, ast.Lambda)):
            for a in node.args.args + node.args.kwonlyargs:
                defined.add(a.arg)
        if isinstance(node, ast.Name) and isinstance(node.ctx, ast.Store):
            defined.add(node.id)
        if isinstance(node, (ast.FunctionDef, ast.ClassDef)):
            defined.add(node.name)
    used = {n.id for n in ast.walk(tree) if isinstance(n, ast.Name) and isinstance(n.ctx, ast.Load)}
    assert used <= defined, sorted(used - defined)
    assert timing.HIP_EVENT_DISABLE_SYSTEM_FENCE == 0x20000000


def test_bench_library_validates_like_the_library():
    """A timed call with fake (never dereferenced) addresses is rejected with
    the same status as the plain call, before any event or launch."""
    from lse_weighted_merge_dcp_amd import timing

    lib = timing.bench_lib()
    args = list(dict(src_o=A, so_R=0, so_B=512, so_H=64, src_lse=A, sl_R=0, sl_B=8, sl_H=1,
                     dst_o=A, do_R=0, do_N=256, do_B=128, do_H=64, dst_lse=A, dl_R=0, dl_N=4, dl_B=2, dl_H=1,
                     kv_len=None, kl_R=0, kl_B=1, R=1, N=3, B=4, H=8, D=64, dtype=0, stream=None).values())
    assert lib.dcpb_pack(A, A + 256, *args, None) == HEADS    # N = 3 does not divide H = 8
    assert _lib.lib().dcp_pack(*args) == HEADS
    args[-6], args[-5] = 2, 0                                  # N = 2, B = 0: a valid no-op
    shape = timing.LaunchShape()
    import ctypes
    assert lib.dcpb_pack(A, A + 256, *args, ctypes.cast(shape.buf, ctypes.c_void_p)) == OK
    assert shape.launches == 0
    assert _lib.lib().dcp_pack(*args) == OK


def test_lse_pack_dim_and_status_strings():
    lib = _lib.lib()
    assert lib.dcp_lse_pack_dim(0) == 1
    assert lib.dcp_lse_pack_dim(1) == 2
    assert lib.dcp_lse_pack_dim(2) == 2
    assert lib.dcp_lse_pack_dim(3) == 4          # OCP FP8 E4M3: 4 bytes / 1 byte
    assert lib.dcp_lse_pack_dim(4) == DTYPE
    assert lib.dcp_lse_pack_dim(-1) == DTYPE
    for code, name in _lib.STATUS.items():
        assert lib.dcp_status_str(code).decode().startswith(name)
    assert ops.lse_pack_dim(torch.float16) == 2
    assert ops.lse_pack_dim(torch.float8_e4m3fn) == 4
    with pytest.raises(ValueError):
        ops.lse_pack_dim(torch.float64)
    with pytest.raises(ValueError):
        ops.lse_pack_dim(torch.float8_e5m2)


def pack(**kw):
    args = dict(src_o=A, so_R=0, so_B=512, so_H=64, src_lse=A, sl_R=0, sl_B=8, sl_H=1,
                dst_o=A, do_R=0, do_N=256, do_B=128, do_H=64, dst_lse=A, dl_R=0, dl_N=4, dl_B=2, dl_H=1,
                kv_len=None, kl_R=0, kl_B=1,
                R=1, N=2, B=4, H=8, D=64, dtype=0, stream=None)
    args.update(kw)
    return _lib.lib().dcp_pack(*args.values())


def combine(**kw):
    args = dict(recv_o=A, ro_R=0, ro_N=4096, ro_B=256, ro_H=64, recv_lse=A, rl_R=0, rl_N=16, rl_B=4, rl_H=1,
                out=A, oo_R=0, oo_B=256, oo_H=64, out_lse=A, ol_R=0, ol_B=4, ol_H=1,
                R=1, N=2, B=4, Hpr=4, D=64, dtype=0, lse_base=0, stream=None)
    args.update(kw)
    return _lib.lib().dcp_unpack_combine(*args.values())


def inplace(**kw):
    args = dict(partial=A, p_N=8192, p_T=512, p_H=64, lse=A, l_N=32, l_T=8, l_H=1, h0=0, h1=4,
                out=A, o_T=256, o_H=64, out_lse=A, ol_T=4, ol_H=1, N=2, P=2, rank0=0, T=4, H=8, D=64,
                dtype=0, lse_base=0, stream=None)
    args.update(kw)
    return _lib.lib().dcp_lse_combine_inplace(*args.values())


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=4), DTYPE), (dict(dtype=-1), DTYPE),
    (dict(N=0), SHAPE), (dict(H=0), SHAPE), (dict(D=0), SHAPE), (dict(B=-1), SHAPE), (dict(R=-1), SHAPE),
    (dict(N=3), HEADS), (dict(N=16), HEADS),
    (dict(so_H=-1), STRIDE), (dict(dl_N=-4), STRIDE), (dict(do_R=-1), STRIDE),
    (dict(src_o=None), NULL), (dict(dst_lse=None), NULL),
    (dict(src_lse=A + 2), ALIGN), (dict(dst_o=A + 1, dtype=1), ALIGN), (dict(dst_o=A + 2, dtype=0), ALIGN),
    (dict(kv_len=A + 2), ALIGN), (dict(kl_B=-1), STRIDE), (dict(kv_len=A, B=0), OK),
    (dict(dst_o=A + 1, dtype=3, B=0), OK), (dict(dst_lse=A + 1, dtype=3), ALIGN),   # fp8: byte-aligned payload
    (dict(D=1 << 28, dtype=3), SHAPE),
    (dict(H=1 << 25, N=1), SHAPE), (dict(D=1 << 27), SHAPE),
    (dict(H=1 << 22, N=1), SHAPE), (dict(H=1 << 11, N=1, D=1 << 20), SHAPE),   # one token's rows > 2^25
    (dict(B=0), OK), (dict(R=0), OK), (dict(B=0, src_o=None), OK),
    # limits that keep host arithmetic inside int64
    (dict(so_B=(1 << 56) + 1), STRIDE), (dict(dl_H=(1 << 63) - 1), STRIDE), (dict(kl_R=1 << 60), STRIDE),
    (dict(so_B=1 << 55, B=1 << 10), STRIDE), (dict(do_R=1 << 50, dl_R=1, R=1 << 12), STRIDE),
    (dict(D=(1 << 63) - 1), SHAPE), (dict(D=(1 << 62) + 1, dtype=2), SHAPE),
    (dict(R=1 << 40, B=1 << 40), SHAPE), (dict(B=(1 << 63) - 1, so_B=0, sl_B=0, do_B=0, dl_B=0), SHAPE),
    (dict(so_B=1 << 56, B=1 << 20, dtype=3), STRIDE),
])
def test_pack_validation(kw, code):
    assert pack(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), DTYPE), (dict(lse_base=2), BASE), (dict(lse_base=-1), BASE),
    (dict(N=0), SHAPE), (dict(Hpr=0), SHAPE), (dict(D=0), SHAPE), (dict(B=-2), SHAPE), (dict(N=1 << 21), SHAPE),
    (dict(Hpr=1 << 22), SHAPE),
    (dict(ro_N=-1), STRIDE), (dict(ol_B=-4), STRIDE),
    (dict(recv_o=None), NULL), (dict(out=None), NULL), (dict(recv_lse=None), NULL),
    (dict(recv_lse=A + 1), ALIGN), (dict(out_lse=A + 2), ALIGN), (dict(out=A + 1, dtype=2), ALIGN),
    (dict(B=0), OK), (dict(R=0, out=None), OK),
    (dict(ro_N=(1 << 56) + 1), STRIDE), (dict(ro_B=1 << 56, B=1 << 5), STRIDE), (dict(D=(1 << 62) + 3), SHAPE),
    (dict(R=1 << 62, ro_R=0, rl_R=0, oo_R=0, ol_R=0), SHAPE),
])
def test_combine_validation(kw, code):
    assert combine(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=9), DTYPE), (dict(lse_base=5), BASE),
    (dict(P=0), SHAPE), (dict(P=3), SHAPE), (dict(rank0=1), SHAPE), (dict(rank0=-1), SHAPE), (dict(T=-1), SHAPE),
    (dict(H=1 << 22), SHAPE),
    (dict(h0=-1), HRANGE), (dict(h0=4, h1=4), HRANGE), (dict(h1=9), HRANGE), (dict(h0=5, h1=3), HRANGE),
    (dict(p_T=-1), STRIDE), (dict(ol_H=-1), STRIDE),
    (dict(partial=None), NULL), (dict(lse=None), NULL),
    (dict(partial=A + 2), ALIGN), (dict(lse=A + 3), ALIGN), (dict(out=A + 2), ALIGN),
    (dict(T=0), OK),
    (dict(rank0=(1 << 63) - 1), SHAPE), (dict(P=(1 << 63) - 1), SHAPE), (dict(N=1 << 62, P=1 << 61), SHAPE),
    (dict(o_T=(1 << 56) + 1), STRIDE), (dict(p_N=1 << 58), STRIDE), (dict(T=1 << 30, p_T=1 << 40), STRIDE),
    (dict(T=1 << 62, p_T=0, l_T=0, o_T=0, ol_T=0), SHAPE), (dict(D=(1 << 63) - 1), SHAPE),
])
def test_inplace_validation(kw, code):
    assert inplace(**kw) == code


def test_binding_rejects_host_tensors_and_bad_layouts():
    out = torch.zeros(2, 8, 64)
    lse = torch.zeros(2, 8)
    with pytest.raises(ValueError):
        ops.dcp_pack_a2a_send(out, lse, torch.zeros(2, 2, 4, 64), torch.zeros(2, 2, 4))
    with pytest.raises(ValueError):
        ops.dcp_lse_combine(torch.zeros(2, 2, 4, 64), torch.zeros(2, 2, 4))
    with pytest.raises(ValueError):
        ops.cp_lse_combine_inplace(torch.zeros(2, 2, 4, 64), torch.zeros(2, 2, 4))
    send = torch.zeros(2, 2, 4, 66, dtype=torch.bfloat16)
    pay, words = ops.interleaved_views(send, 64)
    assert pay.shape == (2, 2, 4, 64) and words.shape == (2, 2, 4) and words.dtype == torch.float32
    assert words.stride() == (2 * 4 * 33, 4 * 33, 33)
    with pytest.raises(ValueError):
        ops.interleaved_views(torch.zeros(2, 2, 4, 65, dtype=torch.bfloat16), 63)
    # fp8: an interleaved row is D + 4 bytes, the LSE is fp32 word D / 4
    send = torch.zeros(2, 2, 4, 68, dtype=torch.float8_e4m3fn)
    pay, words = ops.interleaved_views(send, 64)
    assert pay.shape == (2, 2, 4, 64) and words.shape == (2, 2, 4)
    assert words.stride() == (2 * 4 * 17, 4 * 17, 17)
    assert words.data_ptr() == send.data_ptr() + 64
    with pytest.raises(ValueError):
        ops.interleaved_views(torch.zeros(2, 2, 4, 66, dtype=torch.float8_e4m3fn), 62)
    # empty buffers: any strides (numpy gives zero-size arrays zero strides)
    import numpy as np
    empty = torch.from_numpy(np.zeros((2, 0, 4, 66), np.float16))
    pay, words = ops.interleaved_views(empty, 64)
    assert pay.shape == (2, 0, 4, 64) and words.shape == (2, 0, 4)


FASTDIV_TEST = r"""
#include <cstdio>
#include <cstdint>
#include <random>
#include "fastdiv.hpp"
int main() {
    std::mt19937_64 g(1);
    const uint32_t ds[] = {1u, 2u, 3u, 5u, 7u, 12u, 16u, 96u, 127u, 128u, 129u, 1000u, 4096u, 65535u, 65536u,
                           16777217u, 0x7fffffffu, 0x80000000u, 0x80000001u, 0xfffffffeu, 0xffffffffu};
    long bad = 0;
    for (uint32_t d : ds) {
        dcp::FastDiv f = dcp::make_fastdiv(d);
        const uint32_t edge[] = {0u, 1u, d - 1u, d, d + 1u, 2u * d - 1u, 0x7fffffffu, 0x80000000u, 0xfffffffeu, 0xffffffffu};
        for (uint32_t n : edge) bad += dcp::fdiv(n, f) != n / d;
        for (int i = 0; i < 200000; ++i) { uint32_t n = (uint32_t)g(); bad += dcp::fdiv(n, f) != n / d; }
    }
    for (int i = 0; i < 2000; ++i) {
        uint32_t d = (uint32_t)g() >> (g() % 32); if (d == 0) d = 1;
        dcp::FastDiv f = dcp::make_fastdiv(d);
        for (int k = 0; k < 500; ++k) { uint32_t n = (uint32_t)g(); bad += dcp::fdiv(n, f) != n / d; }
    }
    std::printf("%ld\n", bad);
    return bad != 0;
}
"""


def test_fastdiv_matches_integer_division(tmp_path):
    src = tmp_path / "fd.cpp"
    src.write_text(FASTDIV_TEST)
    exe = str(tmp_path / "fd")
    subprocess.check_call(["g++", "-O2", "-std=c++17", "-I" + CSRC, str(src), "-o", exe])
    r = subprocess.run([exe], capture_output=True, text=True)
    assert r.returncode == 0 and r.stdout.strip() == "0", r.stdout


BLOCK_ORDER_TEST = r"""
#include <cstdio>
#include <cstdint>
#include <vector>
#include "block_order.hpp"
template <uint32_t C>
long check(uint32_t n) {
    std::vector<char> seen(n, 0);
    long bad = 0;
    for (uint32_t b = 0; b < n; ++b) {
        const uint32_t l = dcp::xcd_chunked_order<C>(b, n);
        if (l >= n || seen[l]) ++bad; else seen[l] = 1;
        // the selecting form is the same map
        bad += dcp::xcd_chunked_order_sel<C>(b, n) != l;
    }
    // a grid of at most 8 C blocks keeps the contiguous order
    if (n <= 8 * C)
        for (uint32_t b = 0; b < n; ++b) bad += dcp::xcd_chunked_order<C>(b, n) != dcp::xcd_contiguous_order(b, n);
    return bad;
}
int main() {
    long bad = 0;
    std::vector<uint32_t> ns;
    for (uint32_t n = 1; n <= 5000; ++n) ns.push_back(n);
    for (uint32_t n : {8191u, 8192u, 8193u, 16384u, 16391u, 65536u, 786432u, 786439u, 1u << 21}) ns.push_back(n);
    for (uint32_t n : ns) {
        std::vector<char> seen(n, 0);
        for (uint32_t b = 0; b < n; ++b) {
            const uint32_t l = dcp::xcd_contiguous_order(b, n);
            if (l >= n || seen[l]) ++bad; else seen[l] = 1;
            // consecutive workgroups of one XCD take consecutive blocks
            if (b >= 8 && l != dcp::xcd_contiguous_order(b - 8, n) + 1) ++bad;
        }
        bad += check<1>(n) + check<3>(n) + check<64>(n) + check<128>(n) + check<256>(n) + check<512>(n) +
               check<1024>(n);
    }
    // inside whole rounds, XCD x's k-th workgroup is block k mod C of chunk (k / C) * 8 + x
    for (uint32_t b = 0; b < 16384; ++b) {
        const uint32_t x = b % 8, k = b / 8;
        bad += dcp::xcd_chunked_order<256>(b, 16384) != ((k / 256) * 8 + x) * 256 + k % 256;
    }
    std::printf("%ld\n", bad);
    return bad != 0;
}
"""


def test_block_orders_are_bijections(tmp_path):
    """The XCD-aware workgroup orders (csrc/block_order.hpp, the same code the
    kernels run) map every grid of up to 5000 blocks, and larger ones of the
    workloads' sizes, one to one onto its blocks; the branch-free form of the
    chunked order is the same map."""
    src = tmp_path / "bo.cpp"
    src.write_text(BLOCK_ORDER_TEST)
    exe = str(tmp_path / "bo")
    subprocess.check_call(["g++", "-O2", "-std=c++17", "-I" + CSRC, str(src), "-o", exe])
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.strip() == "0", r.stdout


def test_header_compiles_as_c_and_the_c_client_links(tmp_path):
    """include/dcpmerge.h is plain C: a C11 caller (tests/c_abi_client.c)
    compiles with -Wall -Wextra -Werror and links against libdcpmerge.so and
    the HIP runtime.  Run without arguments it prints its usage and exits
    before any HIP call."""
    import __graft_entry__

    _lib.lib()
    exe = __graft_entry__.build_c_client(str(tmp_path / "client"))
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 1 and "usage" in r.stderr


def test_binding_constants_match_the_header():
    """The dtype, LSE-base and status codes the Python binding passes are the
    values include/dcpmerge.h gives them."""
    text = open(HEADER).read()
    values = {name: int(v) for name, v in re.findall(r"\b(DCP_[A-Z0-9_]+)\s*=\s*(-?\d+)", text)}
    for name in ("DCP_F32", "DCP_F16", "DCP_BF16", "DCP_FP8_E4M3", "DCP_LSE_BASE_E", "DCP_LSE_BASE_2"):
        assert values[name] == getattr(_lib, name), name
    for code, name in _lib.STATUS.items():
        assert values[name] == code, name
    assert sorted(v for k, v in values.items() if k.startswith("DCP_ERR_") or k == "DCP_OK") == sorted(_lib.STATUS)
