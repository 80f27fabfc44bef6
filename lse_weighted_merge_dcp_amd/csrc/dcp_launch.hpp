// dcp_launch.hpp -- internal interface between the C ABI (api.cpp) and the
// kernel launchers.  All strides here are in BYTES; the ABI converts.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fastdiv.hpp"

namespace dcp {

enum DType { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2, DT_FP8 = 3 };

// Bytes per payload element of a DType (0 for anything else).
constexpr int dtype_esize(int dt) {
    return dt == DT_F32 ? 4 : dt == DT_F16 || dt == DT_BF16 ? 2 : dt == DT_FP8 ? 1 : 0;
}

// Timing events a call attaches to its own kernel dispatches (measurement
// only; the library's exported calls never set them).
struct CallTiming {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
    int64_t* shape = nullptr;   // nullable: [launches, workgroups of the last, threads per workgroup]
};

// Pack (and the plain strided row copy the N == 1 shortcuts use):
// for r < R, b < B, h < H with p = h / Hpr, hl = h % Hpr
//   dst[r, p, b, hl, 0:row_bytes] = src[r, b, h, 0:row_bytes]
//   dst_lse[r, p, b, hl]          = src_lse[r, b, h]        (if dst_lse != nullptr)
// dst == nullptr skips the payload.  kv (nullable, int32 per (r, b)): where it
// is 0 the row is sent as the neutral pair (payload 0, LSE -inf).
struct PackArgs {
    const char* src;
    const char* src_lse;
    char* dst;
    char* dst_lse;
    const char* kv = nullptr;
    int64_t kv_R = 0, kv_B = 0;
    int64_t s_R, s_B, s_H;
    int64_t sl_R, sl_B, sl_H;
    int64_t d_R, d_N, d_B, d_H;
    int64_t dl_R, dl_N, dl_B, dl_H;
    int64_t R, B, H, Hpr;
    int64_t row_bytes;
    int esize;
    CallTiming* timing = nullptr;   // nullable: events for this call's dispatches
};

// Out-of-place combine over the peer axis N (see dcp_unpack_combine).
struct CombineArgs {
    const char* recv;
    const char* recv_lse;
    char* out;
    char* out_lse;  // nullable
    int64_t r_R, r_N, r_B, r_H;
    int64_t rl_R, rl_N, rl_B, rl_H;
    int64_t o_R, o_B, o_H;
    int64_t ol_R, ol_B, ol_H;
    int64_t R, N, B, Hpr, D;
    int dtype;
    bool base2;
    CallTiming* timing = nullptr;   // nullable: events for this call's dispatches
};

// In-place merge (see dcp_lse_combine_inplace).
struct InplaceArgs {
    char* partial;
    const char* lse;
    char* out;      // nullable
    char* out_lse;  // nullable
    int64_t p_N, p_T, p_H;
    int64_t l_N, l_T, l_H;
    int64_t o_T, o_H;
    int64_t ol_T, ol_H;
    int64_t N, P, rank0, T, H, D, h0, h1;
    int dtype;
    bool base2;
    CallTiming* timing = nullptr;   // nullable: events for this call's dispatches
};

// Launch kernel(arg) and return that launch's own status.  (Reading the
// thread's last error after a launch would also report, and clear, a stale
// error the caller left from an unrelated call.)  With timing events (t not
// null) the events travel with the dispatch itself, so no marker is added to
// the stream between kernels: `start` goes on the call's first launch only,
// `stop` on every launch, so that it ends up on the last one.
template <typename Arg>
inline hipError_t launch_kernel(void (*kernel)(Arg), dim3 grid, dim3 block, hipStream_t stream, const Arg& arg,
                                CallTiming* t) {
    void* args[] = {const_cast<Arg*>(&arg)};
    if (t != nullptr && t->shape != nullptr) {
        t->shape[0] += 1;
        t->shape[1] = grid.x;
        t->shape[2] = block.x;
    }
    if (t == nullptr || (t->start == nullptr && t->stop == nullptr))
        return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, args, 0, stream);
    hipError_t e = hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, args, 0, stream, t->start,
                                      t->stop, 0);
    t->start = nullptr;
    return e;
}

// Each launcher returns hipSuccess or the launch error; arguments are
// assumed validated by the caller.
hipError_t launch_pack(const PackArgs& a, hipStream_t stream);
hipError_t launch_combine(const CombineArgs& a, hipStream_t stream);
hipError_t launch_inplace(const InplaceArgs& a, hipStream_t stream);

// Largest vector width (16, 8, 4, 2 or 1 bytes, at least esize) such that
// every row length is a multiple of it and every address used is aligned to
// min(width, 4).
int pick_vec_bytes(int64_t row_bytes, int esize, const int64_t* addrs_and_strides, int count);

// Launches are split so that one launch never addresses more than this many
// row-steps (keeps every in-kernel index within 32 bits).
constexpr int64_t kMaxRowsPerLaunch = int64_t(1) << 30;

// The grid size of a launch, counted in work-items, must fit in 32 bits; with
// 256-lane workgroups, at most 2^23 of them per launch (2^31 work-items).
constexpr int64_t kMaxBlocksPerLaunch = int64_t(1) << 23;

// Combine and in-place calls whose merged output spans at least this many
// bytes write it with the nontemporal hint: an output of a quarter of the
// 256 MB Infinity Cache or more cannot stay there for its reader anyway, and
// streaming it out keeps it from evicting the rows still to be read
// (measured: the Kimi-K3-shaped reduce-scatter merge, 402 MB of output,
// 5.4 -> 5.7 TB/s; the long-context B = 64 step, 8 MB of output, 3% slower
// with the hint).
constexpr int64_t kNtOutputBytes = int64_t(64) << 20;

// Row-steps one launch may take when each 256-lane workgroup takes
// units_per_block of them: both limits above hold.
constexpr int64_t max_units_per_launch(int64_t units_per_block) {
    return kMaxBlocksPerLaunch * units_per_block < kMaxRowsPerLaunch ? kMaxBlocksPerLaunch * units_per_block
                                                                     : kMaxRowsPerLaunch;
}

}  // namespace dcp
