// dcp_calls.hpp -- the entry points of libdcpmerge as internal C++ calls that
// also take timing events for their own kernel dispatches.  api.cpp exports
// them without timing (the C ABI of include/dcpmerge.h); the separate
// measurement library (bench_api.cpp) exports them with it.  Arguments and
// status codes are those of include/dcpmerge.h.
#pragma once
#include <stdint.h>

#include "dcp_launch.hpp"

namespace dcp {

// Returned by a call that carries timing events while its stream is being
// captured (nothing enqueued).  Never returned by the exported C ABI, which
// carries no events.
constexpr int kStatusCapture = -10;

int pack_call(const void* src_o, int64_t so_R, int64_t so_B, int64_t so_H,
              const float* src_lse, int64_t sl_R, int64_t sl_B, int64_t sl_H,
              void* dst_o, int64_t do_R, int64_t do_N, int64_t do_B, int64_t do_H,
              float* dst_lse, int64_t dl_R, int64_t dl_N, int64_t dl_B, int64_t dl_H,
              const int32_t* kv_len, int64_t kl_R, int64_t kl_B,
              int64_t R, int64_t N, int64_t B, int64_t H, int64_t D,
              int dtype, void* stream, CallTiming* timing);

int combine_call(const void* recv_o, int64_t ro_R, int64_t ro_N, int64_t ro_B, int64_t ro_H,
                 const float* recv_lse, int64_t rl_R, int64_t rl_N, int64_t rl_B, int64_t rl_H,
                 void* out, int64_t oo_R, int64_t oo_B, int64_t oo_H,
                 float* out_lse, int64_t ol_R, int64_t ol_B, int64_t ol_H,
                 int64_t R, int64_t N, int64_t B, int64_t Hpr, int64_t D,
                 int dtype, int lse_base, void* stream, CallTiming* timing);

int inplace_call(void* partial, int64_t p_N, int64_t p_T, int64_t p_H,
                 const float* lse, int64_t l_N, int64_t l_T, int64_t l_H,
                 int64_t h0, int64_t h1,
                 void* out, int64_t o_T, int64_t o_H,
                 float* out_lse, int64_t ol_T, int64_t ol_H,
                 int64_t N, int64_t P, int64_t rank0,
                 int64_t T, int64_t H, int64_t D,
                 int dtype, int lse_base, void* stream, CallTiming* timing);

}  // namespace dcp
