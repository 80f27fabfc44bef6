// host_launch_check.cpp -- drives libdcpmerge's real host code (api.cpp,
// bench_api.cpp and the launchers of pack.hip, combine.hip and inplace.hip,
// compiled for the host only) with random valid calls, from tiny shapes to
// ones that need several launches, and checks every kernel launch it makes:
// a grid of 1 to 2^23 workgroups of 64, 128, 256 or 512 threads, at most
// 2^31 threads in all (the dispatch packet counts work-items in 32 bits).
// The HIP runtime's launch and registration entry points are replaced by the
// stubs below, so no GPU and no HIP runtime is involved; addresses are fake
// and never dereferenced.  A third of the calls go through the measurement
// library (dcpmerge_bench.h) with timing events: the start event must ride
// on a call's first launch only, the stop event on every launch, and the
// recorded launch shape must count the launches and hold the last one's
// grid.  Built with ASan and UBSan, any overflow in the host arithmetic
// aborts.
//
//   host_launch_check ITERATIONS SEED
//
// Prints "ok <calls> <launches> <most launches in one call> <largest grid in
// work-items>" and exits 0, or reports the first broken expectation and
// exits 1.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cinttypes>
#include <cstdio>
#include <cstdlib>
#include <random>

#include "../include/dcpmerge.h"
#include "../lse_weighted_merge_dcp_amd/csrc/dcpmerge_bench.h"

namespace {
long launches = 0, bad_launch = 0, bad_events = 0;
uint64_t most_items = 0;
uint32_t last_grid = 0, last_block = 0;
// timing events of the launches of the current call, in order
long ext_launches = 0, ext_with_start = 0, ext_first_without_start = 0, ext_without_stop = 0;

void record(dim3 g, dim3 b) {
    ++launches;
    last_grid = g.x;
    last_block = b.x;
    if ((uint64_t)g.x * b.x > most_items) most_items = (uint64_t)g.x * b.x;
    const bool ok = g.x >= 1 && g.x <= (1u << 23) && g.y == 1 && g.z == 1 && b.y == 1 && b.z == 1 &&
                    (b.x == 64 || b.x == 128 || b.x == 256 || b.x == 512) &&
                    (uint64_t)g.x * b.x <= (uint64_t(1) << 31);
    if (!ok) {
        ++bad_launch;
        std::fprintf(stderr, "bad launch: grid %u x %u x %u, block %u x %u x %u\n", g.x, g.y, g.z, b.x, b.y, b.z);
    }
}
}  // namespace

extern "C" {
void** __hipRegisterFatBinary(const void*) {
    static void* handle[1];
    return handle;
}
void __hipRegisterFunction(void**, const void*, char*, const char*, unsigned int, uint3*, uint3*, dim3*, dim3*, int*) {}
void __hipUnregisterFatBinary(void**) {}
hipError_t __hipPopCallConfiguration(dim3*, dim3*, size_t*, hipStream_t*) { return hipSuccess; }
hipError_t hipLaunchKernel(const void*, dim3 g, dim3 b, void**, size_t, hipStream_t) {
    record(g, b);
    return hipSuccess;
}
hipError_t hipExtLaunchKernel(const void*, dim3 g, dim3 b, void**, size_t, hipStream_t, hipEvent_t start,
                              hipEvent_t stop, int) {
    record(g, b);
    if (ext_launches == 0 && start == nullptr) ++ext_first_without_start;
    if (start != nullptr) ++ext_with_start;
    if (stop == nullptr) ++ext_without_stop;
    ++ext_launches;
    return hipSuccess;
}
hipError_t hipStreamIsCapturing(hipStream_t, hipStreamCaptureStatus* s) {
    *s = hipStreamCaptureStatusNone;
    return hipSuccess;
}
}

namespace {
std::mt19937_64 rng;
int64_t pick(std::initializer_list<int64_t> xs) { return xs.begin()[rng() % xs.size()]; }
int64_t small(int64_t hi) { return 1 + (int64_t)(rng() % (uint64_t)hi); }
void* P(int64_t a) { return (void*)(uintptr_t)a; }
void* const EV0 = P(0x10);   // fake timing-event handles
void* const EV1 = P(0x20);
const int64_t A = int64_t(1) << 20;   // fake 1 MiB-aligned base address
int esize(int dt) { return dt == DCP_F32 ? 4 : dt == DCP_FP8_E4M3 ? 1 : 2; }

// a size that is sometimes tiny, sometimes ragged, sometimes huge
int64_t extent(int64_t huge) {
    switch (rng() % 4) {
        case 0: return small(9);
        case 1: return small(std::min<int64_t>(huge, 3000));
        case 2: return std::min(huge, pick({64, 256, 512, 2048, 16384}));
        default: return small(huge);
    }
}

int fail(const char* what, long call) {
    std::fprintf(stderr, "call %ld: %s\n", call, what);
    return 1;
}
}  // namespace

int main(int argc, char** argv) {
    const long iters = argc > 1 ? std::atol(argv[1]) : 20000;
    rng.seed(argc > 2 ? std::strtoull(argv[2], nullptr, 10) : 1);
    long most = 0;
    for (long it = 0; it < iters; ++it) {
        const long before = launches;
        const int dt = (int)(rng() % 4), e = esize(dt);
        const int lpd = 4 / e;
        int st = 0;
        bool idle = false;
        // a third of the calls go through the measurement library with
        // timing events (fake handles: the stubs never dereference them)
        const bool timed = rng() % 3 == 0;
        int64_t shape[3] = {0, 0, 0};
        ext_launches = ext_with_start = ext_first_without_start = ext_without_stop = 0;
        const int which = (int)(rng() % 3);
        if (which == 0) {
            // pack into a peer-outer interleaved buffer [R, N, B, Hpr, D + lpd] (the stream
            // kernel when it applies) or a split-like buffer [R, B, Hpr, N, D] (row kernel)
            const int64_t N = pick({1, 2, 4, 8, 16, 3, 5});
            const int64_t Hpr = pick({1, 2, 3, 8, 12, 16});
            const int64_t H = N * Hpr;
            int64_t D = pick({64, 128, 256, 512, 1024, 2048, 100, 8});
            D = (D + lpd - 1) / lpd * lpd;
            const int64_t R = extent(64), B = extent(int64_t(1) << 22);
            const int64_t W = D + lpd;
            const bool split = rng() % 3 == 0;
            const int64_t so_B = H * D, so_R = B * so_B;
            const int64_t kv = rng() % 4 == 0 ? A : 0;
            if (!split) {
                const int64_t sH = W, sB = Hpr * W, sN = B * sB, sR = N * sN;
                st = timed ? dcpb_pack(EV0, EV1, P(A), so_R, so_B, D, (const float*)P(A), B * H, H, 1, P(A), sR, sN, sB,
                                       sH, (float*)P(A + D * e), sR * e / 4, sN * e / 4, sB * e / 4, sH * e / 4,
                                       (const int32_t*)P(kv), B, 1, R, N, B, H, D, dt, nullptr, shape)
                           : dcp_pack(P(A), so_R, so_B, D, (const float*)P(A), B * H, H, 1, P(A), sR, sN, sB, sH,
                                      (float*)P(A + D * e), sR * e / 4, sN * e / 4, sB * e / 4, sH * e / 4,
                                      (const int32_t*)P(kv), B, 1, R, N, B, H, D, dt, nullptr);
            } else {
                st = timed ? dcpb_pack(EV0, EV1, P(A), so_R, so_B, D, (const float*)P(A), B * H, H, 1, P(A),
                                       B * Hpr * N * D, D, Hpr * N * D, N * D, (float*)P(A), B * Hpr * N * 2, 2,
                                       Hpr * N * 2, N * 2, (const int32_t*)P(kv), B, 1, R, N, B, H, D, dt, nullptr, shape)
                           : dcp_pack(P(A), so_R, so_B, D, (const float*)P(A), B * H, H, 1, P(A), B * Hpr * N * D, D,
                                      Hpr * N * D, N * D, (float*)P(A), B * Hpr * N * 2, 2, Hpr * N * 2, N * 2,
                                      (const int32_t*)P(kv), B, 1, R, N, B, H, D, dt, nullptr);
            }
        } else if (which == 1) {
            // combine N received partials [R, N, B, Hpr, D] (contiguous or interleaved rows)
            const int64_t N = pick({1, 2, 4, 8, 16, 3, 17, 33});
            const int64_t Hpr = pick({1, 3, 8, 12, 16, 96});
            int64_t D = pick({64, 128, 256, 512, 1024, 2048, 100, 8});
            D = (D + lpd - 1) / lpd * lpd;
            const int64_t R = extent(64), B = extent(int64_t(1) << 20);
            const int64_t W = rng() % 2 ? D + lpd : D;
            const int64_t rH = W, rB = Hpr * W, rN = B * rB, rR = N * rN;
            float* ol = (float*)P(rng() % 2 ? A : 0);
            const int base = (int)(rng() % 2);
            st = timed ? dcpb_unpack_combine(EV0, EV1, P(A), rR, rN, rB, rH, (const float*)P(A), N * B * Hpr, B * Hpr,
                                             Hpr, 1, P(A), B * Hpr * D, Hpr * D, D, ol, B * Hpr, Hpr, 1, R, N, B, Hpr,
                                             D, dt, base, nullptr, shape)
                       : dcp_unpack_combine(P(A), rR, rN, rB, rH, (const float*)P(A), N * B * Hpr, B * Hpr, Hpr, 1,
                                            P(A), B * Hpr * D, Hpr * D, D, ol, B * Hpr, Hpr, 1, R, N, B, Hpr, D, dt,
                                            base, nullptr);
        } else {
            // in-place merge of P held partials [P, T, H, D], heads [h0, h1)
            const int64_t N = pick({1, 2, 4, 8, 16, 3, 17});
            const int64_t Pn = rng() % 2 ? N : small(N);
            const int64_t rank0 = (int64_t)(rng() % (uint64_t)(N - Pn + 1));
            const int64_t H = pick({1, 8, 12, 96, 128});
            int64_t D = pick({64, 128, 512, 1024, 100, 8});
            D = (D + lpd - 1) / lpd * lpd;
            const int64_t T = extent(int64_t(1) << 20);
            const int64_t h0 = (int64_t)(rng() % (uint64_t)H), h1 = h0 + 1 + (int64_t)(rng() % (uint64_t)(H - h0));
            void* out = P(rng() % 4 ? A : 0);
            float* out_lse = (float*)P(rng() % 2 ? A : 0);
            idle = N == 1 && !out && !out_lse;
            const int base = (int)(rng() % 2);
            st = timed ? dcpb_lse_combine_inplace(EV0, EV1, P(A), T * H * D, H * D, D, (const float*)P(A), T * H, H, 1,
                                                  h0, h1, out, (h1 - h0) * D, D, out_lse, h1 - h0, 1, N, Pn, rank0, T,
                                                  H, D, dt, base, nullptr, shape)
                       : dcp_lse_combine_inplace(P(A), T * H * D, H * D, D, (const float*)P(A), T * H, H, 1, h0, h1,
                                                 out, (h1 - h0) * D, D, out_lse, h1 - h0, 1, N, Pn, rank0, T, H, D, dt,
                                                 base, nullptr);
        }
        if (st != DCP_OK && st != DCP_ERR_SHAPE) return fail(dcp_status_str(st), it);
        if (bad_launch) return fail("launch outside the limits", it);
        const long n = launches - before;
        // every accepted call launches at least once, except an in-place call
        // with nothing to write (N == 1 and no output)
        if (st == DCP_OK && n == 0 && !(which == 2 && idle)) return fail("accepted call launched nothing", it);
        if (timed) {
            // the start event rides on the call's first launch only, the stop
            // event on every launch; the shape counts the launches and holds
            // the last one's grid
            const bool ok = ext_launches == n && (n == 0 || (ext_with_start == 1 && ext_first_without_start == 0 &&
                                                             ext_without_stop == 0)) &&
                            shape[0] == n && (n == 0 || (shape[1] == last_grid && shape[2] == last_block));
            if (!ok) ++bad_events;
            if (bad_events) return fail("timing events or launch shape not as documented", it);
        } else if (ext_launches != 0) {
            return fail("an untimed call launched with events", it);
        }
        if (n > most) most = n;
    }
    std::printf("ok %ld %ld %ld %" PRIu64 "\n", iters, launches, most, most_items);
    return 0;
}
