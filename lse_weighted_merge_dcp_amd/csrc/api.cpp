// api.cpp -- the C ABI of libdcpmerge (declared in include/dcpmerge.h).
//
// Every check runs on the host before anything is enqueued, so a rejected
// call has no side effect and the error paths run without a GPU.  Element
// and word strides are turned into byte strides for the launchers.  The
// exported calls keep no state: each one is validated, launched and done.
// The internal dcp::*_call functions behind them also take timing events
// for the kernels' own dispatches; only the separate measurement library
// (bench_api.cpp) passes any.
#include <stdint.h>

#include "../../include/dcpmerge.h"
#include "dcp_calls.hpp"
#include "dcp_launch.hpp"

namespace {

using dcp::max_units_per_launch;

int esize_of(int dtype) {
    switch (dtype) {
        case DCP_F32: return 4;
        case DCP_F16: return 2;
        case DCP_BF16: return 2;
        case DCP_FP8_E4M3: return 1;
        default: return 0;
    }
}

bool aligned(const void* p, int a) { return ((uintptr_t)p % (uintptr_t)a) == 0; }

// Limits that keep every size and offset the library computes from its
// arguments inside int64 (and far beyond any device memory): a stride is at
// most 2^56 elements, a view spans less than 2^60 bytes, and a call moves
// at most 2^56 payload bytes.
constexpr int64_t kMaxStride = int64_t(1) << 56;
constexpr int64_t kMaxSpan = int64_t(1) << 60;
constexpr int64_t kMaxCallBytes = int64_t(1) << 56;

bool strides_ok(std::initializer_list<int64_t> xs) {
    for (int64_t x : xs)
        if (x < 0 || x > kMaxStride) return false;
    return true;
}

// The product of non-negative factors is at most `limit` (no overflow).
bool product_le(std::initializer_list<int64_t> xs, int64_t limit) {
    int64_t p = 1;
    for (int64_t x : xs) {
        if (x != 0 && p > limit / x) return false;
        p *= x;
    }
    return p <= limit;
}

// A view of extents n_d and element strides s_d (validated by strides_ok)
// with elements of `esize` bytes spans sum_d (n_d - 1) * s_d * esize bytes;
// true if that stays below kMaxSpan.
struct Dim {
    int64_t n, s;
};
bool span_ok(std::initializer_list<Dim> dims, int64_t esize) {
    int64_t span = 0;
    for (const Dim& d : dims) {
        if (d.n <= 1 || d.s == 0) continue;
        if (d.n - 1 > kMaxSpan / (d.s * esize)) return false;
        span += (d.n - 1) * d.s * esize;
        if (span >= kMaxSpan) return false;
    }
    return true;
}

// The launchers split the work along R, B and T, never inside one token:
// the row-steps of one token (at most H * (row_bytes / 32 + 1) for any
// kernel) must fit in one launch of the kernel with the fewest row-steps per
// workgroup (4), so that every launch stays within its index and grid limits.
bool shape_fits(int64_t H, int64_t D, int64_t esize) {
    if (H > (int64_t(1) << 24) || D > (int64_t(1) << 28) / esize) return false;
    return H * (D * esize / 32 + 1) <= max_units_per_launch(4);
}

int launch_status(hipError_t e) { return e == hipSuccess ? DCP_OK : DCP_ERR_LAUNCH; }

// A call that carries timing events is refused on a capturing stream: the
// events travel with kernel dispatches, which a capture does not record.
int timing_capture_check(const dcp::CallTiming* timing, void* stream) {
    if (timing == nullptr || (timing->start == nullptr && timing->stop == nullptr)) return DCP_OK;
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing((hipStream_t)stream, &st) != hipSuccess) return DCP_ERR_LAUNCH;
    return st == hipStreamCaptureStatusNone ? DCP_OK : dcp::kStatusCapture;
}

}  // namespace

int dcp::pack_call(const void* src_o, int64_t so_R, int64_t so_B, int64_t so_H,
                   const float* src_lse, int64_t sl_R, int64_t sl_B, int64_t sl_H,
                   void* dst_o, int64_t do_R, int64_t do_N, int64_t do_B, int64_t do_H,
                   float* dst_lse, int64_t dl_R, int64_t dl_N, int64_t dl_B, int64_t dl_H,
                   const int32_t* kv_len, int64_t kl_R, int64_t kl_B,
                   int64_t R, int64_t N, int64_t B, int64_t H, int64_t D,
                   int dtype, void* stream, CallTiming* timing) {
    const int e = esize_of(dtype);
    if (e == 0) return DCP_ERR_DTYPE;
    if (R < 0 || B < 0 || N < 1 || H < 1 || D < 1) return DCP_ERR_SHAPE;
    if (H % N != 0) return DCP_ERR_HEADS_NOT_DIVISIBLE;
    if (!shape_fits(H, D, e)) return DCP_ERR_SHAPE;
    if (!strides_ok({so_R, so_B, so_H, sl_R, sl_B, sl_H, do_R, do_N, do_B, do_H, dl_R, dl_N, dl_B, dl_H, kl_R, kl_B}))
        return DCP_ERR_STRIDE;
    if (R == 0 || B == 0) return DCP_OK;
    if (!product_le({R, B, H, D, e}, kMaxCallBytes)) return DCP_ERR_SHAPE;
    const int64_t Hpr = H / N;
    if (!span_ok({{R, so_R}, {B, so_B}, {H, so_H}, {D, 1}}, e) || !span_ok({{R, sl_R}, {B, sl_B}, {H, sl_H}}, 4) ||
        !span_ok({{R, do_R}, {N, do_N}, {B, do_B}, {Hpr, do_H}, {D, 1}}, e) ||
        !span_ok({{R, dl_R}, {N, dl_N}, {B, dl_B}, {Hpr, dl_H}}, 4) || !span_ok({{R, kl_R}, {B, kl_B}}, 4))
        return DCP_ERR_STRIDE;
    if (!src_o || !src_lse || !dst_o || !dst_lse) return DCP_ERR_NULL;
    if (!aligned(src_o, e) || !aligned(dst_o, e) || !aligned(src_lse, 4) || !aligned(dst_lse, 4) ||
        (kv_len && !aligned(kv_len, 4)))
        return DCP_ERR_ALIGN;
    if (int st = timing_capture_check(timing, stream)) return st;
    dcp::PackArgs a;
    a.src = (const char*)src_o;
    a.src_lse = (const char*)src_lse;
    a.dst = (char*)dst_o;
    a.dst_lse = (char*)dst_lse;
    a.s_R = so_R * e; a.s_B = so_B * e; a.s_H = so_H * e;
    a.sl_R = sl_R * 4; a.sl_B = sl_B * 4; a.sl_H = sl_H * 4;
    a.d_R = do_R * e; a.d_N = do_N * e; a.d_B = do_B * e; a.d_H = do_H * e;
    a.dl_R = dl_R * 4; a.dl_N = dl_N * 4; a.dl_B = dl_B * 4; a.dl_H = dl_H * 4;
    a.kv = (const char*)kv_len;
    a.kv_R = kl_R * 4; a.kv_B = kl_B * 4;
    a.R = R; a.B = B; a.H = H; a.Hpr = Hpr;
    a.row_bytes = D * e;
    a.esize = e;
    a.timing = timing;
    return launch_status(dcp::launch_pack(a, (hipStream_t)stream));
}

int dcp::combine_call(const void* recv_o, int64_t ro_R, int64_t ro_N, int64_t ro_B, int64_t ro_H,
                      const float* recv_lse, int64_t rl_R, int64_t rl_N, int64_t rl_B, int64_t rl_H,
                      void* out, int64_t oo_R, int64_t oo_B, int64_t oo_H,
                      float* out_lse, int64_t ol_R, int64_t ol_B, int64_t ol_H,
                      int64_t R, int64_t N, int64_t B, int64_t Hpr, int64_t D,
                      int dtype, int lse_base, void* stream, CallTiming* timing) {
    const int e = esize_of(dtype);
    if (e == 0) return DCP_ERR_DTYPE;
    if (lse_base != DCP_LSE_BASE_E && lse_base != DCP_LSE_BASE_2) return DCP_ERR_LSE_BASE;
    if (R < 0 || B < 0 || N < 1 || Hpr < 1 || D < 1) return DCP_ERR_SHAPE;
    if (N > (int64_t(1) << 20) || !shape_fits(Hpr, D, e)) return DCP_ERR_SHAPE;
    if (!strides_ok({ro_R, ro_N, ro_B, ro_H, rl_R, rl_N, rl_B, rl_H, oo_R, oo_B, oo_H, ol_R, ol_B, ol_H}))
        return DCP_ERR_STRIDE;
    if (R == 0 || B == 0) return DCP_OK;
    if (!product_le({R, N, B, Hpr, D, e}, kMaxCallBytes)) return DCP_ERR_SHAPE;
    if (!span_ok({{R, ro_R}, {N, ro_N}, {B, ro_B}, {Hpr, ro_H}, {D, 1}}, e) ||
        !span_ok({{R, rl_R}, {N, rl_N}, {B, rl_B}, {Hpr, rl_H}}, 4) ||
        !span_ok({{R, oo_R}, {B, oo_B}, {Hpr, oo_H}, {D, 1}}, e) || !span_ok({{R, ol_R}, {B, ol_B}, {Hpr, ol_H}}, 4))
        return DCP_ERR_STRIDE;
    if (!recv_o || !recv_lse || !out) return DCP_ERR_NULL;
    if (!aligned(recv_o, e) || !aligned(out, e) || !aligned(recv_lse, 4) || (out_lse && !aligned(out_lse, 4)))
        return DCP_ERR_ALIGN;
    if (int st = timing_capture_check(timing, stream)) return st;
    if (N == 1) {
        // the world_size == 1 shortcut: out and out_lse are the partial and its LSE, unchanged
        dcp::PackArgs a;
        a.src = (const char*)recv_o;
        a.src_lse = (const char*)recv_lse;
        a.dst = (char*)out;
        a.dst_lse = (char*)out_lse;
        a.s_R = ro_R * e; a.s_B = ro_B * e; a.s_H = ro_H * e;
        a.sl_R = rl_R * 4; a.sl_B = rl_B * 4; a.sl_H = rl_H * 4;
        a.d_R = oo_R * e; a.d_N = 0; a.d_B = oo_B * e; a.d_H = oo_H * e;
        a.dl_R = ol_R * 4; a.dl_N = 0; a.dl_B = ol_B * 4; a.dl_H = ol_H * 4;
        a.R = R; a.B = B; a.H = Hpr; a.Hpr = Hpr;
        a.row_bytes = D * e;
        a.esize = e;
        a.timing = timing;
        return launch_status(dcp::launch_pack(a, (hipStream_t)stream));
    }
    dcp::CombineArgs a;
    a.recv = (const char*)recv_o;
    a.recv_lse = (const char*)recv_lse;
    a.out = (char*)out;
    a.out_lse = (char*)out_lse;
    a.r_R = ro_R * e; a.r_N = ro_N * e; a.r_B = ro_B * e; a.r_H = ro_H * e;
    a.rl_R = rl_R * 4; a.rl_N = rl_N * 4; a.rl_B = rl_B * 4; a.rl_H = rl_H * 4;
    a.o_R = oo_R * e; a.o_B = oo_B * e; a.o_H = oo_H * e;
    a.ol_R = ol_R * 4; a.ol_B = ol_B * 4; a.ol_H = ol_H * 4;
    a.R = R; a.N = N; a.B = B; a.Hpr = Hpr; a.D = D;
    a.dtype = dtype;
    a.base2 = lse_base == DCP_LSE_BASE_2;
    a.timing = timing;
    return launch_status(dcp::launch_combine(a, (hipStream_t)stream));
}

int dcp::inplace_call(void* partial, int64_t p_N, int64_t p_T, int64_t p_H,
                      const float* lse, int64_t l_N, int64_t l_T, int64_t l_H,
                      int64_t h0, int64_t h1,
                      void* out, int64_t o_T, int64_t o_H,
                      float* out_lse, int64_t ol_T, int64_t ol_H,
                      int64_t N, int64_t P, int64_t rank0,
                      int64_t T, int64_t H, int64_t D,
                      int dtype, int lse_base, void* stream, CallTiming* timing) {
    const int e = esize_of(dtype);
    if (e == 0) return DCP_ERR_DTYPE;
    if (lse_base != DCP_LSE_BASE_E && lse_base != DCP_LSE_BASE_2) return DCP_ERR_LSE_BASE;
    if (T < 0 || N < 1 || H < 1 || D < 1 || P < 1 || rank0 < 0) return DCP_ERR_SHAPE;
    if (N > (int64_t(1) << 20) || P > N || rank0 > N - P || !shape_fits(H, D, e)) return DCP_ERR_SHAPE;
    if (h0 < 0 || h1 <= h0 || h1 > H) return DCP_ERR_HEAD_RANGE;
    if (!strides_ok({p_N, p_T, p_H, l_N, l_T, l_H, o_T, o_H, ol_T, ol_H})) return DCP_ERR_STRIDE;
    if (T == 0) return DCP_OK;
    if (!product_le({P, T, H, D, e}, kMaxCallBytes) || !product_le({N, T, H, 4}, kMaxCallBytes))
        return DCP_ERR_SHAPE;
    if (!span_ok({{P, p_N}, {T, p_T}, {H, p_H}, {D, 1}}, e) || !span_ok({{N, l_N}, {T, l_T}, {H, l_H}}, 4) ||
        !span_ok({{T, o_T}, {h1 - h0, o_H}, {D, 1}}, e) || !span_ok({{T, ol_T}, {h1 - h0, ol_H}}, 4))
        return DCP_ERR_STRIDE;
    if (!partial || !lse) return DCP_ERR_NULL;
    if (!aligned(partial, e) || (out && !aligned(out, e)) || !aligned(lse, 4) || (out_lse && !aligned(out_lse, 4)))
        return DCP_ERR_ALIGN;
    if (int st = timing_capture_check(timing, stream)) return st;
    if (N == 1) {
        // the world_size == 1 shortcut: the partial stays as it is; the slice is copied
        if (!out && !out_lse) return DCP_OK;
        dcp::PackArgs a;
        a.src = (const char*)partial + h0 * p_H * e;
        a.src_lse = (const char*)lse + h0 * l_H * 4;
        a.dst = (char*)out;
        a.dst_lse = (char*)out_lse;
        a.s_R = 0; a.s_B = p_T * e; a.s_H = p_H * e;
        a.sl_R = 0; a.sl_B = l_T * 4; a.sl_H = l_H * 4;
        a.d_R = 0; a.d_N = 0; a.d_B = o_T * e; a.d_H = o_H * e;
        a.dl_R = 0; a.dl_N = 0; a.dl_B = ol_T * 4; a.dl_H = ol_H * 4;
        a.R = 1; a.B = T; a.H = h1 - h0; a.Hpr = h1 - h0;
        a.row_bytes = D * e;
        a.esize = e;
        a.timing = timing;
        return launch_status(dcp::launch_pack(a, (hipStream_t)stream));
    }
    dcp::InplaceArgs a;
    a.partial = (char*)partial;
    a.lse = (const char*)lse;
    a.out = (char*)out;
    a.out_lse = (char*)out_lse;
    a.p_N = p_N * e; a.p_T = p_T * e; a.p_H = p_H * e;
    a.l_N = l_N * 4; a.l_T = l_T * 4; a.l_H = l_H * 4;
    a.o_T = o_T * e; a.o_H = o_H * e;
    a.ol_T = ol_T * 4; a.ol_H = ol_H * 4;
    a.N = N; a.P = P; a.rank0 = rank0; a.T = T; a.H = H; a.D = D; a.h0 = h0; a.h1 = h1;
    a.dtype = dtype;
    a.base2 = lse_base == DCP_LSE_BASE_2;
    a.timing = timing;
    return launch_status(dcp::launch_inplace(a, (hipStream_t)stream));
}

extern "C" {

int dcp_lse_pack_dim(int dtype) {
    const int e = esize_of(dtype);
    return e == 0 ? DCP_ERR_DTYPE : 4 / e;
}

const char* dcp_status_str(int status) {
    switch (status) {
        case DCP_OK: return "DCP_OK";
        case DCP_ERR_NULL: return "DCP_ERR_NULL: a required pointer is NULL";
        case DCP_ERR_SHAPE: return "DCP_ERR_SHAPE: invalid or too large extent";
        case DCP_ERR_HEADS_NOT_DIVISIBLE: return "DCP_ERR_HEADS_NOT_DIVISIBLE: H is not a multiple of N";
        case DCP_ERR_DTYPE: return "DCP_ERR_DTYPE: unsupported payload dtype";
        case DCP_ERR_LSE_BASE: return "DCP_ERR_LSE_BASE: lse_base is neither DCP_LSE_BASE_E nor DCP_LSE_BASE_2";
        case DCP_ERR_STRIDE: return "DCP_ERR_STRIDE: negative or too large stride";
        case DCP_ERR_ALIGN: return "DCP_ERR_ALIGN: payload not element-aligned or LSE not 4-byte aligned";
        case DCP_ERR_HEAD_RANGE: return "DCP_ERR_HEAD_RANGE: need 0 <= h0 < h1 <= H";
        case DCP_ERR_LAUNCH: return "DCP_ERR_LAUNCH: HIP kernel launch failed";
        default: return "unknown dcpmerge status";
    }
}

int dcp_pack(const void* src_o, int64_t so_R, int64_t so_B, int64_t so_H,
             const float* src_lse, int64_t sl_R, int64_t sl_B, int64_t sl_H,
             void* dst_o, int64_t do_R, int64_t do_N, int64_t do_B, int64_t do_H,
             float* dst_lse, int64_t dl_R, int64_t dl_N, int64_t dl_B, int64_t dl_H,
             const int32_t* kv_len, int64_t kl_R, int64_t kl_B,
             int64_t R, int64_t N, int64_t B, int64_t H, int64_t D,
             int dtype, void* stream) {
    return dcp::pack_call(src_o, so_R, so_B, so_H, src_lse, sl_R, sl_B, sl_H, dst_o, do_R, do_N, do_B, do_H,
                          dst_lse, dl_R, dl_N, dl_B, dl_H, kv_len, kl_R, kl_B, R, N, B, H, D, dtype, stream,
                          nullptr);
}

int dcp_unpack_combine(const void* recv_o, int64_t ro_R, int64_t ro_N, int64_t ro_B, int64_t ro_H,
                       const float* recv_lse, int64_t rl_R, int64_t rl_N, int64_t rl_B, int64_t rl_H,
                       void* out, int64_t oo_R, int64_t oo_B, int64_t oo_H,
                       float* out_lse, int64_t ol_R, int64_t ol_B, int64_t ol_H,
                       int64_t R, int64_t N, int64_t B, int64_t Hpr, int64_t D,
                       int dtype, int lse_base, void* stream) {
    return dcp::combine_call(recv_o, ro_R, ro_N, ro_B, ro_H, recv_lse, rl_R, rl_N, rl_B, rl_H, out, oo_R, oo_B,
                             oo_H, out_lse, ol_R, ol_B, ol_H, R, N, B, Hpr, D, dtype, lse_base, stream, nullptr);
}

int dcp_lse_combine_inplace(void* partial, int64_t p_N, int64_t p_T, int64_t p_H,
                            const float* lse, int64_t l_N, int64_t l_T, int64_t l_H,
                            int64_t h0, int64_t h1,
                            void* out, int64_t o_T, int64_t o_H,
                            float* out_lse, int64_t ol_T, int64_t ol_H,
                            int64_t N, int64_t P, int64_t rank0,
                            int64_t T, int64_t H, int64_t D,
                            int dtype, int lse_base, void* stream) {
    return dcp::inplace_call(partial, p_N, p_T, p_H, lse, l_N, l_T, l_H, h0, h1, out, o_T, o_H, out_lse, ol_T,
                             ol_H, N, P, rank0, T, H, D, dtype, lse_base, stream, nullptr);
}

}  // extern "C"
