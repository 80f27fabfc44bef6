// fp8_encode_check.hip -- the library's fp8 (OCP E4M3) encoder against a
// table-based nearest-even reference, on every fp32 bit pattern.
//
// The encoder under test is dcp::fp8_e4m3_pack2 (csrc/dcp_device.hpp): the
// payload conversion every kernel uses to round its fp32 results to fp8.  The
// reference is written here from the format's definition: the 127 positive
// finite E4M3 values (code c = 8e + m: m * 2^-9 for e = 0, (1 + m/8) * 2^(e-7)
// otherwise, largest 448) are searched for the neighbours of |f|; the nearer
// one wins, a tie goes to the even code, anything at or beyond 448 (and
// infinity) gives 448, and the sign bit is f's.  Both neighbour gaps are
// exact in fp32 (the neighbours are within a factor of two of |f|), so the
// comparison is exact.  NaN must give one of the two NaN codes.
//
// Thread t (2^24 threads) takes the patterns (i << 24) | t, i = 0..255, and
// encodes each in both halves of the packed word.  Prints the counts per
// input class and exits 0 if no non-NaN pattern differs and every NaN gives
// a NaN code.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>

#include "../lse_weighted_merge_dcp_amd/csrc/dcp_device.hpp"

#define CHECK(x)                                                         \
    do {                                                                 \
        hipError_t e_ = (x);                                             \
        if (e_ != hipSuccess) {                                          \
            printf("%s failed: %s\n", #x, hipGetErrorString(e_));        \
            return 2;                                                    \
        }                                                                \
    } while (0)

__constant__ float kValue[127];   // the positive finite E4M3 values, by code

__device__ uint32_t reference_code(float f) {
    const uint32_t sign = (__float_as_uint(f) >> 24) & 0x80u;
    const float a = fabsf(f);
    if (a >= 448.0f) return sign | 0x7eu;
    // largest code whose value is at most a (kValue is increasing, kValue[0] = 0)
    uint32_t lo = 0, hi = 126;
    while (lo < hi) {
        const uint32_t mid = (lo + hi + 1u) >> 1;
        if (kValue[mid] <= a) lo = mid; else hi = mid - 1u;
    }
    const float below = a - kValue[lo];
    const float above = kValue[lo + 1u] - a;   // lo < 126 since a < 448
    uint32_t c = lo;
    if (above < below || (above == below && (lo & 1u))) c = lo + 1u;
    return sign | c;
}

// classes: 0 = |f| < 448, 1 = 448 <= |f| < 464, 2 = 464 <= |f| <= inf, 3 = NaN
__global__ void compare(unsigned long long* counts) {
    const uint32_t t = blockIdx.x * blockDim.x + threadIdx.x;   // < 2^24 by the launch shape
    uint32_t seen[4] = {0, 0, 0, 0}, bad[4] = {0, 0, 0, 0};
    for (uint32_t i = 0; i < 256u; ++i) {
        const uint32_t u = (i << 24) | t;
        const float f = __uint_as_float(u);
        const uint32_t a = u & 0x7fffffffu;
        const int cls = a > 0x7f800000u ? 3 : (a >= 0x43e80000u ? 2 : (a >= 0x43e00000u ? 1 : 0));
        const uint32_t lo = (uint32_t)dcp::fp8_e4m3_pack2<false>(f, 0.0f, 0) & 0xffu;
        const uint32_t hi = ((uint32_t)dcp::fp8_e4m3_pack2<true>(0.0f, f, 0) >> 24) & 0xffu;
        bool ok;
        if (cls == 3)
            ok = (lo & 0x7fu) == 0x7fu && (hi & 0x7fu) == 0x7fu;
        else
            ok = lo == reference_code(f) && hi == lo;
        seen[cls] += 1u;
        bad[cls] += ok ? 0u : 1u;
    }
    for (int c = 0; c < 4; ++c) {
        atomicAdd(&counts[2 * c], (unsigned long long)seen[c]);
        if (bad[c]) atomicAdd(&counts[2 * c + 1], (unsigned long long)bad[c]);
    }
}

int main() {
    float value[127];
    for (int c = 0; c < 127; ++c) {
        const int e = c >> 3, m = c & 7;
        value[c] = e == 0 ? (float)m / 512.0f : (1.0f + (float)m / 8.0f) * ldexpf(1.0f, e - 7);
    }
    if (value[126] != 448.0f) {
        printf("value table is wrong: largest %g\n", value[126]);
        return 2;
    }
    CHECK(hipMemcpyToSymbol(HIP_SYMBOL(kValue), value, sizeof value));
    unsigned long long* counts = nullptr;
    CHECK(hipMalloc(&counts, 8 * sizeof(unsigned long long)));
    CHECK(hipMemset(counts, 0, 8 * sizeof(unsigned long long)));
    hipLaunchKernelGGL(compare, dim3(1u << 16), dim3(256), 0, 0, counts);   // 2^24 threads
    CHECK(hipGetLastError());
    CHECK(hipDeviceSynchronize());
    unsigned long long c[8];
    CHECK(hipMemcpy(c, counts, sizeof c, hipMemcpyDeviceToHost));
    CHECK(hipFree(counts));
    const char* name[4] = {"below 448", "448 to 464", "464 and beyond", "NaN"};
    unsigned long long total = 0, wrong = 0;
    for (int k = 0; k < 4; ++k) {
        printf("%s: %llu patterns, %llu differ\n", name[k], c[2 * k], c[2 * k + 1]);
        total += c[2 * k];
        wrong += c[2 * k + 1];
    }
    printf("total %llu patterns, %llu differ\n", total, wrong);
    return (total == (1ull << 32) && wrong == 0) ? 0 : 1;
}
