/*
 * dcpmerge_bench.h -- C ABI of libdcpmerge_bench, a measurement library
 * beside libdcpmerge.  Not part of the merge path: the same kernels (built
 * from the same sources), reached through calls that also take two HIP
 * timing events for the call's own kernel dispatches.
 *
 * Why: markers recorded between kernels (hipEventRecord) add a packet, and
 * usually a cache release, to the stream, which stretches the very kernels
 * they time.  Here the events travel with the call's kernel dispatches
 * (hipExtLaunchKernel): `start_event` records when the call's first kernel
 * starts, `stop_event` when its last kernel ends.  Either may be NULL; both
 * NULL is a plain call.  The caller owns the events (hipEvent_t passed as
 * void*, created on the device the call runs on, best with
 * hipEventDisableSystemFence so that no system-scope cache release is added
 * to the timed kernels) and reads them with hipEventElapsedTime.
 *
 * `launch_shape` (nullable, 3 int64 the caller zeroes) receives what the call
 * launched: [0] the number of kernel launches, [1] the workgroups of the
 * last launch, [2] the threads per workgroup of the last launch.
 *
 * Every other argument, the validation and every status code are those of
 * the call of the same name in include/dcpmerge.h, plus one: a call with an
 * event on a stream that is being captured returns DCPB_ERR_CAPTURE and
 * enqueues nothing (a capture does not keep the events).  A call that
 * launches nothing (zero-sized, rejected) leaves both events as they were.
 * The calls keep no state.
 *
 * dcpb_empty_kernel launches a kernel that does nothing, with `blocks`
 * workgroups of `threads` threads (1..1024): the fixed cost of a launch of
 * that shape (dispatch, wave launch and drain), to set beside a timed call.
 */
#ifndef DCPMERGE_BENCH_H
#define DCPMERGE_BENCH_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DCPB_ERR_CAPTURE (-10)

int dcpb_pack(void* start_event, void* stop_event,
              const void* src_o, int64_t so_R, int64_t so_B, int64_t so_H,
              const float* src_lse, int64_t sl_R, int64_t sl_B, int64_t sl_H,
              void* dst_o, int64_t do_R, int64_t do_N, int64_t do_B, int64_t do_H,
              float* dst_lse, int64_t dl_R, int64_t dl_N, int64_t dl_B, int64_t dl_H,
              const int32_t* kv_len, int64_t kl_R, int64_t kl_B,
              int64_t R, int64_t N, int64_t B, int64_t H, int64_t D,
              int dtype, void* stream, int64_t* launch_shape);

int dcpb_unpack_combine(void* start_event, void* stop_event,
                        const void* recv_o, int64_t ro_R, int64_t ro_N, int64_t ro_B, int64_t ro_H,
                        const float* recv_lse, int64_t rl_R, int64_t rl_N, int64_t rl_B, int64_t rl_H,
                        void* out, int64_t oo_R, int64_t oo_B, int64_t oo_H,
                        float* out_lse, int64_t ol_R, int64_t ol_B, int64_t ol_H,
                        int64_t R, int64_t N, int64_t B, int64_t Hpr, int64_t D,
                        int dtype, int lse_base, void* stream, int64_t* launch_shape);

int dcpb_lse_combine_inplace(void* start_event, void* stop_event,
                             void* partial, int64_t p_N, int64_t p_T, int64_t p_H,
                             const float* lse, int64_t l_N, int64_t l_T, int64_t l_H,
                             int64_t h0, int64_t h1,
                             void* out, int64_t o_T, int64_t o_H,
                             float* out_lse, int64_t ol_T, int64_t ol_H,
                             int64_t N, int64_t P, int64_t rank0,
                             int64_t T, int64_t H, int64_t D,
                             int dtype, int lse_base, void* stream, int64_t* launch_shape);

int dcpb_empty_kernel(int64_t blocks, int threads, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DCPMERGE_BENCH_H */
