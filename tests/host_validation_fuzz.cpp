// host_validation_fuzz.cpp -- drives the host side of libdcpmerge's C ABI
// (api.cpp: argument validation and the element-to-byte stride conversion)
// with extreme and random arguments, built with -fsanitize=address,undefined
// so that any overflow or out-of-range arithmetic on the host aborts.  The
// kernel launchers are replaced by stubs that record what they were given,
// so no GPU and no HIP runtime is involved; addresses are fake and never
// dereferenced.
//
//   host_validation_fuzz ITERATIONS SEED
//
// Prints "ok <calls> <accepted>" and exits 0, or reports the first broken
// expectation and exits 1.
#include <cinttypes>
#include <cstdio>
#include <cstdlib>
#include <random>

#include "../include/dcpmerge.h"
#include "../lse_weighted_merge_dcp_amd/csrc/dcp_launch.hpp"

namespace {
int launched = 0;
dcp::PackArgs last_pack;
dcp::CombineArgs last_combine;
dcp::InplaceArgs last_inplace;
}  // namespace

namespace dcp {
hipError_t launch_pack(const PackArgs& a, hipStream_t) { ++launched; last_pack = a; return hipSuccess; }
hipError_t launch_combine(const CombineArgs& a, hipStream_t) { ++launched; last_combine = a; return hipSuccess; }
hipError_t launch_inplace(const InplaceArgs& a, hipStream_t) { ++launched; last_inplace = a; return hipSuccess; }
}  // namespace dcp

extern "C" hipError_t hipStreamIsCapturing(hipStream_t, hipStreamCaptureStatus* s) {
    *s = hipStreamCaptureStatusNone;
    return hipSuccess;
}

namespace {
std::mt19937_64 rng;

int64_t pick() {
    static const int64_t edge[] = {0, 1, 2, 3, 4, 7, 8, 16, 64, 100, 128, 512, 1000, 4096, 65536,
                                   int64_t(1) << 20, int64_t(1) << 24, (int64_t(1) << 24) + 1, int64_t(1) << 28,
                                   (int64_t(1) << 28) + 1, int64_t(1) << 31, int64_t(1) << 32, int64_t(1) << 40,
                                   int64_t(1) << 56, int64_t(1) << 62, INT64_MAX, INT64_MAX - 1, -1, -2,
                                   INT64_MIN, INT64_MIN + 1};
    const int n = sizeof edge / sizeof edge[0];
    switch (rng() % 4) {
        case 0: return edge[rng() % n];
        case 1: return (int64_t)(rng() % 9);
        case 2: return (int64_t)(rng() % 70000);
        default: return (int64_t)rng();
    }
}
int64_t extent() { return rng() % 3 ? (int64_t)(rng() % 17) : pick(); }
int64_t stride() { return rng() % 3 ? (int64_t)(rng() % 5000) : pick(); }
int64_t addr() { return rng() % 8 ? 0x100000 + 256 * (int64_t)(rng() % 4096) + (rng() % 4 ? 0 : (int64_t)(rng() % 4)) : 0; }
int dtype() { return rng() % 8 ? (int)(rng() % 4) : (int)(rng() % 7) - 2; }
int base() { return rng() % 8 ? (int)(rng() % 2) : (int)(rng() % 5) - 2; }
void* P(int64_t a) { return (void*)(uintptr_t)a; }

int fail(const char* what, int call) {
    std::fprintf(stderr, "call %d: %s\n", call, what);
    return 1;
}
}  // namespace

int main(int argc, char** argv) {
    const long iters = argc > 1 ? std::atol(argv[1]) : 100000;
    rng.seed(argc > 2 ? std::strtoull(argv[2], nullptr, 10) : 1);
    long accepted = 0;
    for (long it = 0; it < iters; ++it) {
        const int before = launched;
        int st;
        const int which = (int)(rng() % 3);
        if (which == 0) {
            const int64_t so[3] = {stride(), stride(), stride()}, sl[3] = {stride(), stride(), stride()};
            const int64_t dst_o[4] = {stride(), stride(), stride(), stride()};
            const int64_t dl[4] = {stride(), stride(), stride(), stride()};
            const int64_t kl[2] = {stride(), stride()};
            const int64_t R = extent(), N = extent(), B = extent(), H = extent(), D = extent();
            const int dt = dtype();
            const int64_t kv = rng() % 2 ? addr() : 0;
            st = dcp_pack(P(addr()), so[0], so[1], so[2], (const float*)P(addr()), sl[0], sl[1], sl[2],
                          P(addr()), dst_o[0], dst_o[1], dst_o[2], dst_o[3], (float*)P(addr()), dl[0], dl[1], dl[2],
                          dl[3], (const int32_t*)P(kv), kl[0], kl[1], R, N, B, H, D, dt, nullptr);
            if (st == DCP_OK && launched > before) {
                const dcp::PackArgs& a = last_pack;
                const int e = dt == DCP_F32 ? 4 : dt == DCP_FP8_E4M3 ? 1 : 2;
                if (a.s_B != so[1] * e || a.d_N != dst_o[1] * e || a.dl_H != dl[3] * 4 || a.row_bytes != D * e)
                    return fail("pack: byte strides", (int)it);
                if (a.Hpr * N != H || a.R != R || a.B != B) return fail("pack: extents", (int)it);
            }
        } else if (which == 1) {
            int64_t s[14];
            for (int64_t& x : s) x = stride();
            const int64_t R = extent(), N = extent(), B = extent(), Hpr = extent(), D = extent();
            const int dt = dtype(), bs = base();
            const int64_t olse = rng() % 2 ? addr() : 0;
            st = dcp_unpack_combine(P(addr()), s[0], s[1], s[2], s[3], (const float*)P(addr()), s[4], s[5], s[6], s[7],
                                    P(addr()), s[8], s[9], s[10], (float*)P(olse), s[11], s[12], s[13],
                                    R, N, B, Hpr, D, dt, bs, nullptr);
            if (st == DCP_OK && launched > before && N > 1) {
                const dcp::CombineArgs& a = last_combine;
                const int e = dt == DCP_F32 ? 4 : dt == DCP_FP8_E4M3 ? 1 : 2;
                if (a.r_N != s[1] * e || a.rl_H != s[7] * 4 || a.o_B != s[9] * e || a.D != D)
                    return fail("combine: byte strides", (int)it);
            }
        } else {
            int64_t s[10];
            for (int64_t& x : s) x = stride();
            const int64_t N = extent(), P_ = extent(), rank0 = extent(), T = extent(), H = extent(), D = extent();
            const int64_t h0 = extent(), h1 = extent();
            const int dt = dtype(), bs = base();
            const int64_t out = rng() % 3 ? addr() : 0, olse = rng() % 2 ? addr() : 0;
            st = dcp_lse_combine_inplace(P(addr()), s[0], s[1], s[2], (const float*)P(addr()), s[3], s[4], s[5], h0, h1,
                                         P(out), s[6], s[7], (float*)P(olse), s[8], s[9], N, P_, rank0, T, H, D, dt, bs,
                                         nullptr);
            if (st == DCP_OK && launched > before && N > 1) {
                const dcp::InplaceArgs& a = last_inplace;
                const int e = dt == DCP_F32 ? 4 : dt == DCP_FP8_E4M3 ? 1 : 2;
                if (a.p_T != s[1] * e || a.l_H != s[5] * 4 || a.h1 != h1) return fail("inplace: byte strides", (int)it);
            }
        }
        if (st > 0 || st < DCP_ERR_LAUNCH) return fail("status out of range", (int)it);
        if (st != DCP_OK && launched != before) return fail("rejected call launched", (int)it);
        if (st == DCP_OK) ++accepted;
        if (dcp_status_str(st) == nullptr) return fail("no status text", (int)it);
    }
    std::printf("ok %ld %ld\n", iters, accepted);
    return 0;
}
