/*
 * dcp_oracle.c -- plain, slow, fp64 CPU reference of the DCP partial-merge path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load or call this file's library.  It shares
 * no code, header, table or helper with the HIP library, and the HIP library
 * never calls it.
 *
 * Sources (the pages are PR reports; they print Python, not kernels):
 *   [P1] sglang PR #34651 report, "[DCP] Share one pack kernel between both a2a
 *        backends": section 实现拆解 items 1-3 (head->peer routing, stride-driven
 *        pack, interleaved LSE word, peer-inside split layout) and the code
 *        excerpt of test_pack_serves_the_split_peer_inside_layout.
 *   [P2] vLLM PR #41160 report: section 功能与动机 (exact LSE-weighted reduction)
 *        and 实现拆解 items 1-3 (pack/unpack-combine, is_lse_base_on_e).
 *   [P3] sglang PR #33926 report: 实现拆解 items 3-4 (ranks without KV emit the
 *        neutral pair (0, -inf); LSE base 2 vs base e at the merge site).
 *   [P4] sglang PR #34213 report: code excerpt of cp_lse_ag_out_rs_mha
 *        (world_size == 1 shortcut, logsumexp over the rank axis,
 *        scale = nan_to_num(exp(lse - global_lse)), nan_to_num_ on the partial,
 *        in-place multiply, sum over ranks, head slice).
 *
 * Arithmetic is fp64 throughout.  Parallelism is OpenMP over independent
 * output rows only; the arithmetic inside one row runs in the order the
 * definition states (peer 0, 1, ..., N-1).
 *
 * Every function here is pinned by tests that do not re-type its formulas:
 * a library logsumexp, closed forms, hand-derived fixtures, P1's own
 * view/permute construction of the layouts, and brute-force softmax attention
 * split over KV chunks.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_API __attribute__((visibility("default")))

/* ------------------------------------------------------------------------ */
/* Pack.  [P1] 实现拆解 item 1: head h goes to peer p = h / Hpr as local head  */
/* hl = h % Hpr; the payload row and the fp32 LSE word are copied bit for bit */
/* to dst_o[p, b, hl, :] and dst_lse[p, b, hl].  Every stride is in BYTES.    */
/* Bytes of the destination that no (b, h) addresses are left as they were   */
/* ([P1] 实现拆解 item 3: stats slot 1 is never written).                    */
/* kv_len (nullable, int32 per token, stride kl_b bytes): a token for which  */
/* this rank owns no KV is sent as the neutral pair instead -- payload 0 and */
/* LSE -inf ([P3] 实现拆解 item 3, fixup_zero_kv_rows).                       */
/* ------------------------------------------------------------------------ */
ORC_API void orc_pack(const uint8_t* src_o, int64_t so_b, int64_t so_h, int64_t so_d,
                      const uint8_t* src_lse, int64_t sl_b, int64_t sl_h,
                      uint8_t* dst_o, int64_t do_n, int64_t do_b, int64_t do_h, int64_t do_d,
                      uint8_t* dst_lse, int64_t dl_n, int64_t dl_b, int64_t dl_h,
                      const uint8_t* kv_len, int64_t kl_b,
                      int64_t N, int64_t B, int64_t H, int64_t D, int64_t esize) {
    int64_t Hpr = H / N;
    const float neg_inf = -INFINITY;
    for (int64_t b = 0; b < B; ++b) {
        int32_t len = 1;
        if (kv_len) memcpy(&len, kv_len + b * kl_b, 4);
        for (int64_t h = 0; h < H; ++h) {
            int64_t p = h / Hpr;
            int64_t hl = h % Hpr;
            if (len == 0) {
                for (int64_t d = 0; d < D; ++d)
                    memset(dst_o + p * do_n + b * do_b + hl * do_h + d * do_d, 0, (size_t)esize);
                memcpy(dst_lse + p * dl_n + b * dl_b + hl * dl_h, &neg_inf, 4);
                continue;
            }
            for (int64_t d = 0; d < D; ++d) {
                memcpy(dst_o + p * do_n + b * do_b + hl * do_h + d * do_d,
                       src_o + b * so_b + h * so_h + d * so_d, (size_t)esize);
            }
            memcpy(dst_lse + p * dl_n + b * dl_b + hl * dl_h, src_lse + b * sl_b + h * sl_h, 4);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Global LSE of one row, with the semantics of the torch.logsumexp call in */
/* [P4]'s code excerpt: the running maximum m is replaced by 0 when it is   */
/* +-inf, so any +inf gives +inf, all -inf give -inf, and NaN propagates.   */
/* Base 2 ([P3] 实现拆解 item 4) is the same sum taken with powers of two.   */
/* ------------------------------------------------------------------------ */
static double orc_pow_base(double x, int base2) { return base2 ? exp2(x) : exp(x); }
static double orc_log_base(double x, int base2) { return base2 ? log2(x) : log(x); }

static double orc_global_lse(const double* l, int64_t n, int64_t stride, int base2) {
    double m = -INFINITY;
    for (int64_t i = 0; i < n; ++i) {
        double v = l[i * stride];
        if (isnan(v)) return NAN; /* max() propagates NaN */
        if (v > m) m = v;
    }
    if (isinf(m)) m = 0.0; /* torch masks an infinite maximum to 0 before shifting */
    double s = 0.0;
    for (int64_t i = 0; i < n; ++i) s += orc_pow_base(l[i * stride] - m, base2);
    return m + orc_log_base(s, base2);
}

/* nan_to_num(x, nan=0, posinf=0, neginf=0)  ([P4] code excerpt) */
static double orc_guard(double x) { return isfinite(x) ? x : 0.0; }

/* ------------------------------------------------------------------------ */
/* Out-of-place combine over the peer axis ([P1] 实现拆解 item 3 receive side,*/
/* [P2] 实现拆解 item 1 unpack-combine), per output row:                     */
/*   G   = logsumexp_i l_i   (base e or 2)                                   */
/*   w_i = nan_to_num(base^(l_i - G))                                        */
/*   out = sum_i w_i * nan_to_num(o_i)                                       */
/* The guards are the ones [P4] spells out; N == 1 returns the single        */
/* partial unchanged ([P4] world_size == 1 shortcut).                        */
/*   o   : [N][rows][D] fp64, contiguous;   l : [N][rows] fp64               */
/*   out : [rows][D];  g : [rows];  mag : [rows][D] = sum_i w_i*|o'_i|       */
/*   weights (nullable) : [N][rows]                                          */
/* ------------------------------------------------------------------------ */
ORC_API void orc_combine(const double* o, const double* l, int64_t N, int64_t rows, int64_t D,
                         int base2, double* out, double* g, double* mag, double* weights) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        if (N == 1) {
            g[r] = l[r];
            for (int64_t d = 0; d < D; ++d) {
                out[r * D + d] = o[r * D + d];
                mag[r * D + d] = fabs(o[r * D + d]);
            }
            if (weights) weights[r] = 1.0;
            continue;
        }
        double G = orc_global_lse(l + r, N, rows, base2);
        g[r] = G;
        for (int64_t d = 0; d < D; ++d) {
            out[r * D + d] = 0.0;
            mag[r * D + d] = 0.0;
        }
        for (int64_t i = 0; i < N; ++i) {
            double w = orc_guard(orc_pow_base(l[i * rows + r] - G, base2));
            if (weights) weights[i * rows + r] = w;
            const double* oi = o + (i * rows + r) * D;
            for (int64_t d = 0; d < D; ++d) {
                double x = orc_guard(oi[d]);
                out[r * D + d] += w * x;
                mag[r * D + d] += w * fabs(x);
            }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* In-place merge ([P4] code excerpt): the same G and w_i; every partial is  */
/* overwritten with s_i = nan_to_num(o_i) * w_i, and the merged row is the   */
/* sum of the s_i over the ranks (the all_reduce).  Only P of the N ranks'   */
/* partials may be held (partial j belongs to rank rank0 + j); the sum is    */
/* then over the held ones.  N == 1 leaves the partial untouched.            */
/*   o      : [P][rows][D];  l : [N][rows]                                   */
/*   scaled : [P][rows][D] (the expected partial after the call)             */
/*   out, mag : [rows][D];  g : [rows]                                       */
/* ------------------------------------------------------------------------ */
ORC_API void orc_inplace(const double* o, const double* l, int64_t N, int64_t P, int64_t rank0,
                         int64_t rows, int64_t D, int base2, double* scaled, double* out,
                         double* g, double* mag) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        if (N == 1) {
            g[r] = l[r];
            for (int64_t d = 0; d < D; ++d) {
                scaled[r * D + d] = o[r * D + d];
                out[r * D + d] = o[r * D + d];
                mag[r * D + d] = fabs(o[r * D + d]);
            }
            continue;
        }
        double G = orc_global_lse(l + r, N, rows, base2);
        g[r] = G;
        for (int64_t d = 0; d < D; ++d) {
            out[r * D + d] = 0.0;
            mag[r * D + d] = 0.0;
        }
        for (int64_t j = 0; j < P; ++j) {
            double w = orc_guard(orc_pow_base(l[(rank0 + j) * rows + r] - G, base2));
            const double* oj = o + (j * rows + r) * D;
            double* sj = scaled + (j * rows + r) * D;
            for (int64_t d = 0; d < D; ++d) {
                double x = orc_guard(oj[d]);
                sj[d] = x * w;
                out[r * D + d] += sj[d];
                mag[r * D + d] += fabs(sj[d]);
            }
        }
    }
}

/* Threads the parallel loops use from now on (n >= 1); for timing only. */
ORC_API void orc_set_num_threads(int n) {
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* Thread count OpenMP will use (reported with the CPU baseline). */
ORC_API int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
