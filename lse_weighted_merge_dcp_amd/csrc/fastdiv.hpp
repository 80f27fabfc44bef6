// fastdiv.hpp -- unsigned 32-bit division by a run-time invariant divisor.
//
// q = floor(n / d) for 0 <= n < 2^32, 1 <= d < 2^32, computed as
//   q = (mulhi(n, m) + n) >> s,  s = ceil(log2 d),  m = floor(2^32 (2^s - d) / d) + 1
// (the "round-up" method of Granlund & Montgomery, "Division by invariant
// integers using multiplication", PLDI 1994).  The sum is formed in 64 bits,
// so no overflow correction is needed.  Plain C++: the same code runs on the
// host (where it is unit-tested) and on the GPU (v_mul_hi_u32 / s_mul_hi_u32).
#pragma once
#include <stdint.h>

#if defined(__HIPCC__)
#define DCP_HD __host__ __device__ __forceinline__
#else
#define DCP_HD inline
#endif

namespace dcp {

struct FastDiv {
    uint32_t d;  // divisor
    uint32_t m;  // magic multiplier
    uint32_t s;  // shift
};

inline FastDiv make_fastdiv(uint32_t d) {
    FastDiv f;
    f.d = d;
    uint32_t s = 0;
    while (s < 32 && (uint64_t(1) << s) < d) ++s;
    f.s = s;
    f.m = (uint32_t)(((uint64_t(1) << 32) * ((uint64_t(1) << s) - d)) / d + 1);
    return f;
}

DCP_HD uint32_t fdiv(uint32_t n, FastDiv f) {
    uint32_t hi = (uint32_t)(((uint64_t)n * f.m) >> 32);
    return (uint32_t)(((uint64_t)hi + n) >> f.s);
}

}  // namespace dcp
