/* c_abi_client.c -- a plain C caller of libdcpmerge (no Python, no torch).
 *
 * It shows that the C ABI of include/dcpmerge.h is usable on its own: the
 * program allocates device memory with the HIP runtime, creates its own
 * stream, and runs the decode path of the DCP merge for N ranks stacked in
 * one GPU's memory -- one dcp_pack of every rank into peer-outer interleaved
 * send buffers, then one dcp_unpack_combine of every destination reading the
 * send buffers through transposed strides (the exchange as a zero-copy view).
 *
 *   c_abi_client DIR
 *
 * DIR/meta.txt holds "N B H D dtype lse_base" (dtype and base as the
 * dcp_dtype / dcp_lse_base codes); DIR/out.bin the partials [N, B, H, D] in
 * the payload type; DIR/lse.bin the LSEs [N, B, H] fp32.  Written: DIR/send.bin
 * (the send buffers [N src, N peer, B, H/N, D + lpd]), DIR/comb.bin (the
 * merged rows [N dst, B, H/N, D]) and DIR/g.bin (the global LSE [N, B, H/N]).
 * The caller checks them against the oracle.  The combine is timed with two
 * HIP events recorded around it on the stream (printed as "timed combine:
 * ... us").  Exit status 0 on success.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../include/dcpmerge.h"

#define HIP_OK(x)                                                                  \
    do {                                                                           \
        hipError_t e_ = (x);                                                       \
        if (e_ != hipSuccess) {                                                    \
            fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));         \
            exit(2);                                                               \
        }                                                                          \
    } while (0)

static void* read_file(const char* dir, const char* name, size_t bytes) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE* f = fopen(path, "rb");
    if (!f) { fprintf(stderr, "cannot open %s\n", path); exit(3); }
    void* p = malloc(bytes ? bytes : 1);
    if (fread(p, 1, bytes, f) != bytes) { fprintf(stderr, "short read %s\n", path); exit(3); }
    fclose(f);
    return p;
}

static void write_file(const char* dir, const char* name, const void* p, size_t bytes) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE* f = fopen(path, "wb");
    if (!f || fwrite(p, 1, bytes, f) != bytes) { fprintf(stderr, "cannot write %s\n", path); exit(3); }
    fclose(f);
}

int main(int argc, char** argv) {
    if (argc != 2) { fprintf(stderr, "usage: %s DIR\n", argv[0]); return 1; }
    const char* dir = argv[1];
    char path[4096];
    snprintf(path, sizeof path, "%s/meta.txt", dir);
    FILE* mf = fopen(path, "r");
    long long N, B, H, D;
    int dtype, base;
    if (!mf || fscanf(mf, "%lld %lld %lld %lld %d %d", &N, &B, &H, &D, &dtype, &base) != 6) {
        fprintf(stderr, "bad %s\n", path);
        return 1;
    }
    fclose(mf);

    const int lpd = dcp_lse_pack_dim(dtype);
    if (lpd < 0) { fprintf(stderr, "dcp_lse_pack_dim: %s\n", dcp_status_str(lpd)); return 1; }
    const int e = 4 / lpd;                 /* element size */
    const long long Hpr = H / N, W = D + lpd;
    if ((D * e) % 4 != 0) { fprintf(stderr, "D * e must be a multiple of 4\n"); return 1; }

    const size_t out_bytes = (size_t)(N * B * H * D) * e;
    const size_t lse_bytes = (size_t)(N * B * H) * 4;
    const size_t send_bytes = (size_t)(N * N * B * Hpr * W) * e;
    const size_t comb_bytes = (size_t)(N * B * Hpr * D) * e;
    const size_t g_bytes = (size_t)(N * B * Hpr) * 4;
    void* h_out = read_file(dir, "out.bin", out_bytes);
    void* h_lse = read_file(dir, "lse.bin", lse_bytes);

    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));
    void *d_out, *d_lse, *d_send, *d_comb, *d_g;
    HIP_OK(hipMalloc(&d_out, out_bytes));
    HIP_OK(hipMalloc(&d_lse, lse_bytes));
    HIP_OK(hipMalloc(&d_send, send_bytes));
    HIP_OK(hipMalloc(&d_comb, comb_bytes));
    HIP_OK(hipMalloc(&d_g, g_bytes));
    HIP_OK(hipMemcpy(d_out, h_out, out_bytes, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_lse, h_lse, lse_bytes, hipMemcpyHostToDevice));

    /* a rejected call returns its status and enqueues nothing */
    int st = dcp_pack(NULL, 0, 0, 0, (const float*)d_lse, 0, 0, 0, d_send, 0, 0, 0, 0,
                      (float*)d_send, 0, 0, 0, 0, NULL, 0, 0, 1, N, B, H, D, dtype, stream);
    if (st != DCP_ERR_NULL) { fprintf(stderr, "expected DCP_ERR_NULL, got %d\n", st); return 1; }
    printf("rejected call: %s\n", dcp_status_str(st));

    /* pack: every rank r writes send[r] = [N peer, B, Hpr, W]; the LSE is
     * fp32 word D/lpd of each row, so its strides are the element strides
     * times e/4 and its base pointer is the payload base plus D*e bytes */
    const long long sN = B * Hpr * W, sB = Hpr * W, sH = W, sR = N * sN;
    float* d_words = (float*)((char*)d_send + D * e);
    st = dcp_pack(d_out, B * H * D, H * D, D,
                  (const float*)d_lse, B * H, H, 1,
                  d_send, sR, sN, sB, sH,
                  d_words, sR * e / 4, sN * e / 4, sB * e / 4, sH * e / 4,
                  NULL, 0, 0,
                  N, N, B, H, D, dtype, stream);
    if (st != DCP_OK) { fprintf(stderr, "dcp_pack: %s\n", dcp_status_str(st)); return 1; }

    /* combine: destination p reads send[:, p] -- axes (dst, src) swapped */
    hipEvent_t ev0, ev1;
    HIP_OK(hipEventCreate(&ev0));
    HIP_OK(hipEventCreate(&ev1));
    HIP_OK(hipEventRecord(ev0, stream));
    st = dcp_unpack_combine(d_send, sN, sR, sB, sH,
                            d_words, sN * e / 4, sR * e / 4, sB * e / 4, sH * e / 4,
                            d_comb, B * Hpr * D, Hpr * D, D,
                            (float*)d_g, B * Hpr, Hpr, 1,
                            N, N, B, Hpr, D, dtype, base, stream);
    if (st != DCP_OK) { fprintf(stderr, "dcp_unpack_combine: %s\n", dcp_status_str(st)); return 1; }
    HIP_OK(hipEventRecord(ev1, stream));
    HIP_OK(hipStreamSynchronize(stream));
    float ms = 0.0f;
    HIP_OK(hipEventElapsedTime(&ms, ev0, ev1));
    if (!(ms > 0.0f)) { fprintf(stderr, "timed combine: %g ms\n", ms); return 1; }
    printf("timed combine: %.3f us\n", ms * 1e3);
    HIP_OK(hipEventDestroy(ev0));
    HIP_OK(hipEventDestroy(ev1));

    void* h_send = malloc(send_bytes);
    void* h_comb = malloc(comb_bytes);
    void* h_g = malloc(g_bytes);
    HIP_OK(hipMemcpy(h_send, d_send, send_bytes, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(h_comb, d_comb, comb_bytes, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(h_g, d_g, g_bytes, hipMemcpyDeviceToHost));
    write_file(dir, "send.bin", h_send, send_bytes);
    write_file(dir, "comb.bin", h_comb, comb_bytes);
    write_file(dir, "g.bin", h_g, g_bytes);

    HIP_OK(hipFree(d_out));
    HIP_OK(hipFree(d_lse));
    HIP_OK(hipFree(d_send));
    HIP_OK(hipFree(d_comb));
    HIP_OK(hipFree(d_g));
    HIP_OK(hipStreamDestroy(stream));
    free(h_out); free(h_lse); free(h_send); free(h_comb); free(h_g);
    printf("ok N=%lld B=%lld H=%lld D=%lld dtype=%d base=%d\n", N, B, H, D, dtype, base);
    return 0;
}
