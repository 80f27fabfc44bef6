// bench_api.cpp -- C ABI of libdcpmerge_bench (dcpmerge_bench.h): the
// entry points of include/dcpmerge.h with HIP timing events carried on the
// call's own kernel dispatches.  Measurement only; linked into its own
// library so that libdcpmerge itself stays stateless and event-free.
#include <stdint.h>

#include "dcp_calls.hpp"
#include "dcpmerge_bench.h"

static_assert(DCPB_ERR_CAPTURE == dcp::kStatusCapture, "capture status");

namespace {
dcp::CallTiming events(void* start_event, void* stop_event, int64_t* shape) {
    dcp::CallTiming t;
    t.start = (hipEvent_t)start_event;
    t.stop = (hipEvent_t)stop_event;
    t.shape = shape;
    return t;
}

__global__ __launch_bounds__(1024) void empty_kernel() {}
}  // namespace

extern "C" {

int dcpb_pack(void* start_event, void* stop_event,
              const void* src_o, int64_t so_R, int64_t so_B, int64_t so_H,
              const float* src_lse, int64_t sl_R, int64_t sl_B, int64_t sl_H,
              void* dst_o, int64_t do_R, int64_t do_N, int64_t do_B, int64_t do_H,
              float* dst_lse, int64_t dl_R, int64_t dl_N, int64_t dl_B, int64_t dl_H,
              const int32_t* kv_len, int64_t kl_R, int64_t kl_B,
              int64_t R, int64_t N, int64_t B, int64_t H, int64_t D,
              int dtype, void* stream, int64_t* launch_shape) {
    dcp::CallTiming t = events(start_event, stop_event, launch_shape);
    return dcp::pack_call(src_o, so_R, so_B, so_H, src_lse, sl_R, sl_B, sl_H, dst_o, do_R, do_N, do_B, do_H,
                          dst_lse, dl_R, dl_N, dl_B, dl_H, kv_len, kl_R, kl_B, R, N, B, H, D, dtype, stream, &t);
}

int dcpb_unpack_combine(void* start_event, void* stop_event,
                        const void* recv_o, int64_t ro_R, int64_t ro_N, int64_t ro_B, int64_t ro_H,
                        const float* recv_lse, int64_t rl_R, int64_t rl_N, int64_t rl_B, int64_t rl_H,
                        void* out, int64_t oo_R, int64_t oo_B, int64_t oo_H,
                        float* out_lse, int64_t ol_R, int64_t ol_B, int64_t ol_H,
                        int64_t R, int64_t N, int64_t B, int64_t Hpr, int64_t D,
                        int dtype, int lse_base, void* stream, int64_t* launch_shape) {
    dcp::CallTiming t = events(start_event, stop_event, launch_shape);
    return dcp::combine_call(recv_o, ro_R, ro_N, ro_B, ro_H, recv_lse, rl_R, rl_N, rl_B, rl_H, out, oo_R, oo_B,
                             oo_H, out_lse, ol_R, ol_B, ol_H, R, N, B, Hpr, D, dtype, lse_base, stream, &t);
}

int dcpb_lse_combine_inplace(void* start_event, void* stop_event,
                             void* partial, int64_t p_N, int64_t p_T, int64_t p_H,
                             const float* lse, int64_t l_N, int64_t l_T, int64_t l_H,
                             int64_t h0, int64_t h1,
                             void* out, int64_t o_T, int64_t o_H,
                             float* out_lse, int64_t ol_T, int64_t ol_H,
                             int64_t N, int64_t P, int64_t rank0,
                             int64_t T, int64_t H, int64_t D,
                             int dtype, int lse_base, void* stream, int64_t* launch_shape) {
    dcp::CallTiming t = events(start_event, stop_event, launch_shape);
    return dcp::inplace_call(partial, p_N, p_T, p_H, lse, l_N, l_T, l_H, h0, h1, out, o_T, o_H, out_lse, ol_T,
                             ol_H, N, P, rank0, T, H, D, dtype, lse_base, stream, &t);
}

int dcpb_empty_kernel(int64_t blocks, int threads, void* stream) {
    if (blocks < 1 || blocks > (int64_t(1) << 31) - 1 || threads < 1 || threads > 1024) return -2;
    void* args[] = {nullptr};
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(empty_kernel), dim3((uint32_t)blocks),
                                         dim3((uint32_t)threads), args, 0, (hipStream_t)stream);
    return e == hipSuccess ? 0 : -9;
}

}  // extern "C"
