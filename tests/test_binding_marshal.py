"""The Python binding's marshalling (ops.py), checked on the CPU: a stub
library with the C ABI's entry points records the arguments each call
receives, and the test compares them with the pointers, element strides and
sizes the tensors imply.  Unbatched calls pass R = 1 with zero R strides;
batched and transposed inputs pass their own strides; errors in shapes,
dtypes or layouts raise ValueError before any call."""
import ctypes
import os
import subprocess

import pytest
import torch

from lse_weighted_merge_dcp_amd import _lib, ops

STUB = r"""
#include <stdint.h>
#include <string.h>
static int64_t rec[32];
static int nrec;
#define R(i, v) rec[i] = (int64_t)(v)
int dcp_pack(const void* a0, int64_t a1, int64_t a2, int64_t a3, const void* a4, int64_t a5, int64_t a6, int64_t a7,
             void* a8, int64_t a9, int64_t a10, int64_t a11, int64_t a12, void* a13, int64_t a14, int64_t a15,
             int64_t a16, int64_t a17, const void* a18, int64_t a19, int64_t a20, int64_t a21, int64_t a22,
             int64_t a23, int64_t a24, int64_t a25, int a26, void* a27) {
    R(0, a0); R(1, a1); R(2, a2); R(3, a3); R(4, a4); R(5, a5); R(6, a6); R(7, a7); R(8, a8); R(9, a9);
    R(10, a10); R(11, a11); R(12, a12); R(13, a13); R(14, a14); R(15, a15); R(16, a16); R(17, a17);
    R(18, a18); R(19, a19); R(20, a20); R(21, a21); R(22, a22); R(23, a23); R(24, a24); R(25, a25);
    R(26, a26); R(27, a27); nrec = 28; return 0;
}
int dcp_unpack_combine(const void* a0, int64_t a1, int64_t a2, int64_t a3, int64_t a4, const void* a5,
                       int64_t a6, int64_t a7, int64_t a8, int64_t a9, void* a10, int64_t a11, int64_t a12,
                       int64_t a13, void* a14, int64_t a15, int64_t a16, int64_t a17, int64_t a18, int64_t a19,
                       int64_t a20, int64_t a21, int64_t a22, int a23, int a24, void* a25) {
    R(0, a0); R(1, a1); R(2, a2); R(3, a3); R(4, a4); R(5, a5); R(6, a6); R(7, a7); R(8, a8); R(9, a9);
    R(10, a10); R(11, a11); R(12, a12); R(13, a13); R(14, a14); R(15, a15); R(16, a16); R(17, a17);
    R(18, a18); R(19, a19); R(20, a20); R(21, a21); R(22, a22); R(23, a23); R(24, a24); R(25, a25);
    nrec = 26; return 0;
}
int dcp_lse_combine_inplace(void* a0, int64_t a1, int64_t a2, int64_t a3, const void* a4, int64_t a5,
                            int64_t a6, int64_t a7, int64_t a8, int64_t a9, void* a10, int64_t a11,
                            int64_t a12, void* a13, int64_t a14, int64_t a15, int64_t a16, int64_t a17,
                            int64_t a18, int64_t a19, int64_t a20, int64_t a21, int a22, int a23, void* a24) {
    R(0, a0); R(1, a1); R(2, a2); R(3, a3); R(4, a4); R(5, a5); R(6, a6); R(7, a7); R(8, a8); R(9, a9);
    R(10, a10); R(11, a11); R(12, a12); R(13, a13); R(14, a14); R(15, a15); R(16, a16); R(17, a17);
    R(18, a18); R(19, a19); R(20, a20); R(21, a21); R(22, a22); R(23, a23); R(24, a24);
    nrec = 25; return 0;
}
int dcp_lse_pack_dim(int dt) { return dt == 0 ? 1 : dt == 1 || dt == 2 ? 2 : dt == 3 ? 4 : -2; }
const char* dcp_status_str(int s) { return "stub"; }
int stub_args(int64_t* out) { memcpy(out, rec, sizeof(rec)); return nrec; }
"""


@pytest.fixture
def stub(tmp_path, monkeypatch):
    src = tmp_path / "stub.c"
    src.write_text(STUB)
    so = str(tmp_path / "libstub.so")
    subprocess.check_call(["gcc", "-O1", "-shared", "-fPIC", str(src), "-o", so])
    h = ctypes.CDLL(so)
    for name, (args, res) in _lib.SIGNATURES.items():
        fn = getattr(h, name)
        fn.argtypes = args
        fn.restype = res
    monkeypatch.setattr(_lib, "_lib", h)
    # device-only pieces: CPU tensors stand for device 0, stream 0x5a
    monkeypatch.setattr(ops, "_on_gpu", lambda *ts: 0)
    monkeypatch.setattr(ops, "_stream", lambda dev: 0x5a)
    monkeypatch.setattr(torch.cuda, "current_device", lambda: 0)

    def args():
        buf = (ctypes.c_int64 * 32)()
        n = h.stub_args(buf)
        return list(buf[:n])
    return args


def ptr(t):
    return t.data_ptr()


def test_pack_unbatched_and_batched(stub):
    B, H, D, N = 3, 8, 64, 4
    out = torch.zeros(B, H, D, dtype=torch.bfloat16)
    lse = torch.zeros(B, H)
    send = torch.zeros(N, B, H // N, D + 2, dtype=torch.bfloat16)
    pay, words = ops.interleaved_views(send, D)
    ops.dcp_pack_a2a_send(out, lse, pay, words)
    a = stub()
    assert a == [ptr(out), 0, H * D, D, ptr(lse), 0, H, 1,
                 ptr(pay), 0, B * (H // N) * (D + 2), (H // N) * (D + 2), D + 2,
                 ptr(words), 0, B * (H // N) * (D + 2) // 2, (H // N) * (D + 2) // 2, (D + 2) // 2,
                 0, 0, 0, 1, N, B, H, D, _lib.DCP_BF16, 0x5a]
    # batched over R = 2, with the tokens of the source transposed to [H, B] order
    Rn = 2
    outT = torch.zeros(Rn, H, B, D, dtype=torch.bfloat16).transpose(1, 2)
    lseT = torch.zeros(Rn, H, B).transpose(1, 2)
    sendR = torch.zeros(Rn, N, B, H // N, D + 2, dtype=torch.bfloat16)
    payR, wordsR = ops.interleaved_views(sendR, D)
    kv = torch.ones(Rn, B, dtype=torch.int32)
    ops.dcp_pack_a2a_send(outT, lseT, payR, wordsR, kv_len=kv)
    a = stub()
    assert a[:4] == [ptr(outT), H * B * D, D, B * D]
    assert a[4:8] == [ptr(lseT), H * B, 1, B]
    assert a[18:21] == [ptr(kv), B, 1]
    assert a[21:26] == [Rn, N, B, H, D]


def test_pack_rejects_bad_arguments(stub):
    B, H, D, N = 3, 8, 64, 4
    out = torch.zeros(B, H, D, dtype=torch.bfloat16)
    lse = torch.zeros(B, H)
    send = torch.zeros(N, B, H // N, D + 2, dtype=torch.bfloat16)
    pay, words = ops.interleaved_views(send, D)
    bad = [
        dict(lse=torch.zeros(B, H + 1)),                                   # lse shape
        dict(lse=torch.zeros(B, H, dtype=torch.float16)),                  # lse dtype
        dict(out=torch.zeros(B, H, D)),                                    # payload dtype differs
        dict(out=torch.zeros(B, H, 2 * D, dtype=torch.bfloat16)[..., ::2]),  # D not contiguous
        dict(out=torch.zeros(B, H, D, dtype=torch.float64), dst_o=pay.to(torch.float64)),  # dtype
        dict(dst_o=pay[:3]),                                               # N does not divide H
        dict(dst_lse=words[:, :, :1]),                                     # dst_lse shape
        dict(kv_len=torch.ones(B, dtype=torch.int64)),                     # kv_len dtype
        dict(kv_len=torch.ones(B + 1, dtype=torch.int32)),                 # kv_len shape
        dict(kv_len=torch.ones(1, B, dtype=torch.int32)),                  # kv_len rank vs unbatched call
        dict(out=out[None], lse=lse),                                      # mixed batching
    ]
    for kw in bad:
        args = dict(out=out, lse=lse, dst_o=pay, dst_lse=words)
        args.update(kw)
        with pytest.raises(ValueError):
            ops.dcp_pack_a2a_send(args["out"], args["lse"], args["dst_o"], args["dst_lse"], kv_len=args.get("kv_len"))


def test_combine_unbatched_batched_and_outputs(stub):
    N, B, Hpr, D = 4, 3, 2, 64
    recv = torch.zeros(N, B, Hpr, D, dtype=torch.float16)
    rl = torch.zeros(N, B, Hpr)
    o, g = ops.dcp_lse_combine(recv, rl, is_lse_base_on_e=False)
    a = stub()
    assert o.shape == (B, Hpr, D) and g.shape == (B, Hpr)
    assert a == [ptr(recv), 0, B * Hpr * D, Hpr * D, D, ptr(rl), 0, B * Hpr, Hpr, 1,
                 ptr(o), 0, Hpr * D, D, ptr(g), 0, Hpr, 1, 1, N, B, Hpr, D, _lib.DCP_F16,
                 _lib.DCP_LSE_BASE_2, 0x5a]
    o2, g2 = ops.dcp_lse_combine(recv, rl, return_lse=False)
    a = stub()
    assert g2 is None and a[14:18] == [0, 0, 0, 0] and a[24] == _lib.DCP_LSE_BASE_E
    # batched: peers and ranks transposed, caller's outputs
    Rn = 2
    recvR = torch.zeros(N, Rn, B, Hpr, D, dtype=torch.float16).transpose(0, 1)
    rlR = torch.zeros(N, Rn, B, Hpr).transpose(0, 1)
    oR = torch.zeros(Rn, B, Hpr, D, dtype=torch.float16)
    gR = torch.zeros(Rn, B, Hpr)
    out, gg = ops.dcp_lse_combine(recvR, rlR, out=oR, out_lse=gR)
    a = stub()
    assert out.data_ptr() == oR.data_ptr() and gg.data_ptr() == gR.data_ptr()
    assert a[1:5] == [B * Hpr * D, Rn * B * Hpr * D, Hpr * D, D]
    assert a[6:10] == [B * Hpr, Rn * B * Hpr, Hpr, 1]
    assert a[18:23] == [Rn, N, B, Hpr, D]
    for kw in (dict(out=torch.zeros(B, Hpr, D)),                         # dtype
               dict(out=torch.zeros(B, Hpr + 1, D, dtype=torch.float16)),  # shape
               dict(out=torch.zeros(1, B, Hpr, D, dtype=torch.float16)),   # rank
               dict(out_lse=torch.zeros(B, Hpr + 1)),
               dict(out_lse=torch.zeros(B, Hpr, dtype=torch.float16))):
        with pytest.raises(ValueError):
            ops.dcp_lse_combine(recv, rl, **kw)
    with pytest.raises(ValueError):
        ops.dcp_lse_combine(recv, rl[:, :, :1])


def test_inplace_arguments(stub):
    P, N, T, H, D = 2, 4, 5, 6, 32
    part = torch.zeros(P, T, H, D)
    lse = torch.zeros(N, T, H)
    o = ops.cp_lse_combine_inplace(part, lse, h0=2, h1=5, rank0=1, is_lse_base_on_e=False)
    a = stub()
    assert o.shape == (T, 3, D)
    assert a == [ptr(part), T * H * D, H * D, D, ptr(lse), T * H, H, 1, 2, 5,
                 ptr(o), 3 * D, D, 0, 0, 0, N, P, 1, T, H, D, _lib.DCP_F32, _lib.DCP_LSE_BASE_2, 0x5a]
    o, g = ops.cp_lse_combine_inplace(part, lse, return_lse=True)
    a = stub()
    assert a[8:10] == [0, H] and a[13:16] == [ptr(g), H, 1]
    none = ops.cp_lse_combine_inplace(part, lse, want_out=False)
    a = stub()
    assert none is None and a[10:13] == [0, 0, 0]
    for kw in (dict(out=torch.zeros(T, H + 1, D)), dict(out_lse=torch.zeros(T, H + 1))):
        with pytest.raises(ValueError):
            ops.cp_lse_combine_inplace(part, lse, return_lse="out_lse" in kw, **kw)
    with pytest.raises(ValueError):
        ops.cp_lse_combine_inplace(part, lse[:, :, :1])
