/*
 * dcpmerge.h -- C ABI of libdcpmerge, the decode-context-parallel (DCP)
 * attention partial-merge path on AMD Instinct MI355X (gfx950).
 *
 * Under DCP every rank attends over its own slice of the KV cache and returns
 * a partial output o_r [B, H, D] with its log-sum-exp lse_r [B, H] (fp32).
 * The partials are exchanged and merged by LSE weighting.  This library holds
 * the three data-parallel steps of that path:
 *
 *   dcp_pack                 scatter o_r and lse_r into per-peer send layouts
 *   dcp_unpack_combine       merge N received partials out of place
 *   dcp_lse_combine_inplace  scale the partial buffer in place and sum it
 *
 * Conventions shared by every entry point
 *   - All pointers are device memory owned by the caller.  The library never
 *     allocates, frees, zero-fills, synchronises or copies to the host, so the
 *     calls can be captured in a HIP graph.
 *   - Work is enqueued only on `stream` (a hipStream_t passed as void*; NULL is
 *     the null stream).  The stream and every pointer belong to the calling
 *     thread's current HIP device (hipSetDevice).  Calls keep no state
 *     between them, so calls on different streams may run concurrently.
 *   - Payload tensors hold `dtype` elements; the innermost (D) dimension is
 *     contiguous.  Every other stride is given in ELEMENTS of that tensor's
 *     own type: payload strides in payload elements, LSE strides in fp32
 *     words.  Strides must be >= 0 and at most 2^56, and each view must span
 *     less than 2^60 bytes; otherwise DCP_ERR_STRIDE.
 *   - Payload pointers must be aligned to the element size and LSE pointers
 *     to 4 bytes.  Faster kernels are chosen when the payload rows are
 *     4-byte aligned and D * element size is a multiple of 16 bytes.
 *   - Outputs must not overlap inputs (except where stated) or each other.
 *     Stated exception: the out of dcp_unpack_combine may exactly alias
 *     recv_o's peer 0 rows (same address and strides), merging in place into
 *     the first received partial; out_lse must never alias recv_lse.
 *   - Errors are detected on the host before anything is enqueued: on any
 *     error nothing is written.  A zero-sized call (R, B or T = 0) is DCP_OK.
 *   - Size limits: the heads of one token (H, or Hpr for the combine) times
 *     (D * element size / 32 + 1) must not exceed 2^25, H <= 2^24,
 *     D * element size <= 2^28 bytes, and one call moves at most 2^56
 *     payload bytes; otherwise DCP_ERR_SHAPE.  Within that, R, B and T are
 *     limited only by memory: the library splits them over several
 *     launches.  (These limits keep every size and offset the library
 *     computes inside int64; no device holds memory near them.)
 *   - Leading dimension R ("R independent problems") is an extension for
 *     running several ranks' calls in one launch, e.g. all N simulated ranks
 *     stacked in one GPU's memory.  R = 1 is the single call the pages
 *     describe; R > 1 behaves exactly like R separate calls.
 */
#ifndef DCPMERGE_H
#define DCPMERGE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of the partial outputs.  LSEs are always fp32.
 * DCP_FP8_E4M3 is the OCP FP8 E4M3 format (e4m3fn: bias 7, 3 mantissa bits,
 * subnormals, S.1111.111 = NaN, no infinities, largest finite 448).  The
 * pages mention fp8 only as a future dtype whose word alignment would need
 * review (sglang PR #34651 report, 风险与影响) and which the vLLM helper
 * rejects (vLLM PR #41160 report, 风险与影响); here it follows the same
 * rules as the other types: lpd = 4 / element size = 4, so an interleaved
 * row is D + 4 bytes and needs D % 4 == 0 to keep its LSE word aligned, and
 * merged outputs are rounded to nearest even in fp8. */
typedef enum { DCP_F32 = 0, DCP_F16 = 1, DCP_BF16 = 2, DCP_FP8_E4M3 = 3 } dcp_dtype;

/* Base of the LSE values.  Attention kernels differ (trtllm-gen emits base 2,
 * cute-dsl natural log), so the base is a flag of the merge itself
 * (sglang PR #33926 report, 实现拆解 item 4 and 关联脉络 #34240).
 * The returned global LSE is in the same base as the inputs. */
typedef enum { DCP_LSE_BASE_E = 0, DCP_LSE_BASE_2 = 1 } dcp_lse_base;

/* Status codes.  0 = success, negative = error (nothing enqueued). */
enum {
    DCP_OK = 0,
    DCP_ERR_NULL = -1,                /* a required pointer is NULL                         */
    DCP_ERR_SHAPE = -2,               /* bad extent, P/rank0 out of range, index too large  */
    DCP_ERR_HEADS_NOT_DIVISIBLE = -3, /* dcp_pack: H % N != 0                               */
    DCP_ERR_DTYPE = -4,               /* dtype is not a dcp_dtype                           */
    DCP_ERR_LSE_BASE = -5,            /* lse_base is not a dcp_lse_base                     */
    DCP_ERR_STRIDE = -6,              /* a stride negative or too large, a view too long    */
    DCP_ERR_ALIGN = -7,               /* payload not element-aligned, LSE not 4-byte aligned */
    DCP_ERR_HEAD_RANGE = -8,          /* in-place: not 0 <= h0 < h1 <= H                    */
    DCP_ERR_LAUNCH = -9               /* the HIP kernel launch failed                       */
};

/* Number of payload elements one fp32 LSE occupies when it is interleaved at
 * the tail of a payload row: 1 for DCP_F32, 2 for DCP_F16 and DCP_BF16, 4 for
 * DCP_FP8_E4M3 (vLLM PR #41160 report, 实现拆解 item 2: 4 bytes over the
 * element size; bf16 is 2 like fp16).  Returns DCP_ERR_DTYPE for anything
 * else. */
int dcp_lse_pack_dim(int dtype);

/* Static, human-readable text of a status code. */
const char* dcp_status_str(int status);

/*
 * dcp_pack -- stride-driven pack of one rank's partial for the all-to-all
 * (sglang PR #34651 report, 实现拆解 items 1-3).
 *
 * For every r < R, b < B, h < H, with Hpr = H / N, p = h / Hpr, hl = h % Hpr:
 *   dst_o  [r, p, b, hl, 0:D] = src_o  [r, b, h, 0:D]     (bit copy)
 *   dst_lse[r, p, b, hl]      = src_lse[r, b, h]          (bit copy of the fp32 word)
 * Head h goes to peer p as its local head hl: contiguous head blocks per peer.
 * Because the destination is described only by strides, one call serves both
 * layouts of the pages:
 *   - peer-outer interleaved send buffer S [N, B, Hpr, D + lpd] of dtype:
 *     dst_o = S, strides (B*Hpr*W, Hpr*W, W) with W = D + lpd;
 *     dst_lse = the fp32 word D / lpd of each row: pointer (float*)S + D/lpd,
 *     strides (B*Hpr*W/lpd, Hpr*W/lpd, W/lpd) words.
 *   - peer-inside split layout partial_o [B, Hpr, N, D] and stats
 *     [B, Hpr, N, 2] fp32: dst_o strides (D, Hpr*N*D, N*D) for (N, B, Hpr);
 *     dst_lse = stats slot 0 with word strides (2, Hpr*N*2, N*2).
 * Bytes the map does not address are left untouched, e.g. stats slot 1
 * (the page allocates it with empty() because nothing ever reads it).
 *
 * kv_len (nullable) holds the rank-local KV length of every (r, b) as int32.
 * Where it is 0 the rank owns no KV for that token, and the pack sends the
 * neutral pair instead of the partial: payload 0 and LSE -inf for all H heads
 * (the fixup_zero_kv_rows pass of sglang PR #33926 report, 实现拆解 item 3,
 * fused into the pack).  Non-zero lengths change nothing.  src_o and src_lse
 * are still read for every (r, b, h), zero-KV tokens included (the length is
 * read while the rows are in flight, and their bytes are then dropped), so
 * they must be readable device memory for every token.
 *
 * Strides: src_o (so_R, so_B, so_H) elements; src_lse (sl_R, sl_B, sl_H)
 * words; dst_o (do_R, do_N, do_B, do_H) elements; dst_lse (dl_R, dl_N, dl_B,
 * dl_H) words; kv_len (kl_R, kl_B) int32 elements.  Errors: DCP_ERR_NULL,
 * _SHAPE (R, B < 0; N, H, D < 1), _HEADS_NOT_DIVISIBLE, _DTYPE, _STRIDE,
 * _ALIGN (also kv_len not 4-byte aligned), _LAUNCH.
 */
int dcp_pack(const void* src_o, int64_t so_R, int64_t so_B, int64_t so_H,
             const float* src_lse, int64_t sl_R, int64_t sl_B, int64_t sl_H,
             void* dst_o, int64_t do_R, int64_t do_N, int64_t do_B, int64_t do_H,
             float* dst_lse, int64_t dl_R, int64_t dl_N, int64_t dl_B, int64_t dl_H,
             const int32_t* kv_len, int64_t kl_R, int64_t kl_B,
             int64_t R, int64_t N, int64_t B, int64_t H, int64_t D,
             int dtype, void* stream);

/*
 * dcp_unpack_combine -- LSE-weighted merge of the N received partials, out of
 * place (sglang PR #34651 report, 实现拆解 item 3 receive side; vLLM PR #41160
 * report, 实现拆解 item 1; the guards of sglang PR #34213 report's excerpt).
 *
 * For every r < R, b < B, hl < Hpr, with beta = e or 2 and l_i = recv_lse[r,i,b,hl]:
 *   G     = log_beta sum_i beta^(l_i)         (logsumexp semantics: any NaN -> NaN,
 *                                              else any +inf -> +inf, all -inf -> -inf)
 *   w_i   = nan_to_num(beta^(l_i - G))         (NaN and +-inf become 0)
 *   out[r, b, hl, :]  = sum_i w_i * nan_to_num(recv_o[r, i, b, hl, :])
 *   out_lse[r, b, hl] = G                      (skipped if out_lse is NULL)
 * Accumulation is fp32; out is rounded to nearest even in dtype.  A neutral
 * partial (0, -inf), the pair a rank without KV emits, contributes nothing.
 * N == 1 copies the partial and its LSE unchanged, with no guard
 * (the world_size == 1 shortcut).  The result is deterministic: fixed peer
 * order, no atomics.
 *
 * recv_o may be any strided view [R, N, B, Hpr, D] (e.g. the permuted views of
 * the split layout, or one destination's slice of a stacked send buffer).
 * Over the head slice [h0, h1) of an [N, T, H, D] partial stack (B = T,
 * Hpr = h1 - h0) it is the reduce-scatter flavour of dcp_lse_combine_inplace:
 * the same out and out_lse, with the partials left untouched;
 * strides (ro_R, ro_N, ro_B, ro_H) elements; recv_lse (rl_R, rl_N, rl_B, rl_H)
 * words; out (oo_R, oo_B, oo_H) elements; out_lse (ol_R, ol_B, ol_H) words.
 * Errors: DCP_ERR_NULL, _SHAPE, _DTYPE, _LSE_BASE, _STRIDE, _ALIGN, _LAUNCH.
 */
int dcp_unpack_combine(const void* recv_o, int64_t ro_R, int64_t ro_N, int64_t ro_B, int64_t ro_H,
                       const float* recv_lse, int64_t rl_R, int64_t rl_N, int64_t rl_B, int64_t rl_H,
                       void* out, int64_t oo_R, int64_t oo_B, int64_t oo_H,
                       float* out_lse, int64_t ol_R, int64_t ol_B, int64_t ol_H,
                       int64_t R, int64_t N, int64_t B, int64_t Hpr, int64_t D,
                       int dtype, int lse_base, void* stream);

/*
 * dcp_lse_combine_inplace -- the in-place merge of sglang PR #34213 report
 * (code excerpt of cp_lse_ag_out_rs_mha): the partial buffer is reused for
 * the scaled partials instead of a second [T, H, D] temporary.
 *
 * lse [N, T, H] holds every rank's LSE (the all-gathered stack).  partial
 * [P, T, H, D] holds P of the ranks' partials: partial[j] is rank rank0 + j
 * (P = N, rank0 = 0 when all ranks are stacked on one GPU; P = 1 when a rank
 * holds only its own).  With G and w_i as in dcp_unpack_combine:
 *   partial[j, t, h, :] <- nan_to_num(partial[j, t, h, :]) * w_{rank0+j}   (all t, h)
 *   out[t, h - h0, :]    = sum_j partial[j, t, h, :]  for h in [h0, h1)     (if out != NULL)
 *   out_lse[t, h - h0]   = G[t, h]                    for h in [h0, h1)     (if out_lse != NULL)
 * With P = N, out is the merged result for heads [h0, h1) (the all-reduce
 * followed by the rank's head slice); with P < N it is these ranks' share of
 * that sum.  N == 1 leaves partial untouched and copies the slice.  The
 * caller's partial is overwritten: it is dead after the merge.
 *
 * Strides: partial (p_N, p_T, p_H) elements for (j, t, h); lse (l_N, l_T,
 * l_H) words; out (o_T, o_H) elements; out_lse (ol_T, ol_H) words.
 * Errors: DCP_ERR_NULL, _SHAPE (also P < 1 or rank0 + P > N), _DTYPE,
 * _LSE_BASE, _STRIDE, _ALIGN, _HEAD_RANGE, _LAUNCH.
 */
int dcp_lse_combine_inplace(void* partial, int64_t p_N, int64_t p_T, int64_t p_H,
                            const float* lse, int64_t l_N, int64_t l_T, int64_t l_H,
                            int64_t h0, int64_t h1,
                            void* out, int64_t o_T, int64_t o_H,
                            float* out_lse, int64_t ol_T, int64_t ol_H,
                            int64_t N, int64_t P, int64_t rank0,
                            int64_t T, int64_t H, int64_t D,
                            int dtype, int lse_base, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DCPMERGE_H */
