// dcp_device.hpp -- device helpers shared by the pack, combine and in-place
// kernels: vector memory access, payload conversions, 16-lane DPP row
// reductions and broadcasts, and the XCD-aware block order.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "block_order.hpp"
#include "fastdiv.hpp"

namespace dcp {

// --------------------------------------------------------------------------
// memory access: V-byte vectors at 4-byte (V >= 4) or 2-byte (V == 2)
// alignment.  The payload rows of an interleaved send buffer start 4 bytes
// apart modulo 16, so the vector types only promise dword alignment; gfx950
// serves dword-aligned dwordx2/dwordx4 accesses directly.
// --------------------------------------------------------------------------
typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x2_a4 __attribute__((ext_vector_type(2), aligned(4)));

template <int V> struct Vec;
template <> struct Vec<16> { uint32_t w[4]; };
template <> struct Vec<8>  { uint32_t w[2]; };
template <> struct Vec<4>  { uint32_t w[1]; };
template <> struct Vec<2>  { uint16_t h; };
template <> struct Vec<1>  { uint8_t b; };

template <int V> __device__ __forceinline__ Vec<V> vload(const char* p);
template <> __device__ __forceinline__ Vec<16> vload<16>(const char* p) {
    u32x4_a4 x = *reinterpret_cast<const u32x4_a4*>(p);
    Vec<16> v; v.w[0] = x.x; v.w[1] = x.y; v.w[2] = x.z; v.w[3] = x.w; return v;
}
template <> __device__ __forceinline__ Vec<8> vload<8>(const char* p) {
    u32x2_a4 x = *reinterpret_cast<const u32x2_a4*>(p);
    Vec<8> v; v.w[0] = x.x; v.w[1] = x.y; return v;
}
template <> __device__ __forceinline__ Vec<4> vload<4>(const char* p) {
    Vec<4> v; v.w[0] = *reinterpret_cast<const uint32_t*>(p); return v;
}
template <> __device__ __forceinline__ Vec<2> vload<2>(const char* p) {
    Vec<2> v; v.h = *reinterpret_cast<const uint16_t*>(p); return v;
}
template <> __device__ __forceinline__ Vec<1> vload<1>(const char* p) {
    Vec<1> v; v.b = *reinterpret_cast<const uint8_t*>(p); return v;
}

template <int V> __device__ __forceinline__ Vec<V> vzero() {
    Vec<V> v{};
    return v;
}

template <int V> __device__ __forceinline__ void vstore(char* p, const Vec<V>& v);
template <> __device__ __forceinline__ void vstore<16>(char* p, const Vec<16>& v) {
    u32x4_a4 x; x.x = v.w[0]; x.y = v.w[1]; x.z = v.w[2]; x.w = v.w[3];
    *reinterpret_cast<u32x4_a4*>(p) = x;
}
template <> __device__ __forceinline__ void vstore<8>(char* p, const Vec<8>& v) {
    u32x2_a4 x; x.x = v.w[0]; x.y = v.w[1];
    *reinterpret_cast<u32x2_a4*>(p) = x;
}
template <> __device__ __forceinline__ void vstore<4>(char* p, const Vec<4>& v) {
    *reinterpret_cast<uint32_t*>(p) = v.w[0];
}
template <> __device__ __forceinline__ void vstore<2>(char* p, const Vec<2>& v) {
    *reinterpret_cast<uint16_t*>(p) = v.h;
}
template <> __device__ __forceinline__ void vstore<1>(char* p, const Vec<1>& v) {
    *reinterpret_cast<uint8_t*>(p) = v.b;
}

// A wave-uniform address held in scalar registers: loads from it plus a
// 32-bit per-lane offset take the scalar-base form of the global load (one
// VGPR of offset for any number of rows, no 64-bit address arithmetic per
// lane).  p must be the same for every lane of the wave.
__device__ __forceinline__ uint64_t wave_addr(const char* p) {
    const uint64_t a = (uint64_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// 16 bytes at base + off (global memory, 4-byte aligned); NTL marks the line
// as read once.
typedef const u32x4_a4 __attribute__((address_space(1))) g_u32x4_a4;
template <bool NTL>
__device__ __forceinline__ Vec<16> gload16(uint64_t base, uint32_t off) {
    g_u32x4_a4* p = (g_u32x4_a4*)(base + off);
    u32x4_a4 x;
    if constexpr (NTL) x = __builtin_nontemporal_load(p); else x = *p;
    Vec<16> v;
    v.w[0] = x.x; v.w[1] = x.y; v.w[2] = x.z; v.w[3] = x.w;
    return v;
}

// V bytes at base + off (V = 16 or 4; 4-byte aligned), as gload16.
typedef const uint32_t __attribute__((address_space(1))) g_u32;
template <int V, bool NTL>
__device__ __forceinline__ Vec<V> gloadv(uint64_t base, uint32_t off) {
    if constexpr (V == 16) {
        return gload16<NTL>(base, off);
    } else {
        static_assert(V == 4, "gloadv: V = 16 or 4");
        g_u32* p = (g_u32*)(base + off);
        Vec<4> v;
        if constexpr (NTL) v.w[0] = __builtin_nontemporal_load(p); else v.w[0] = *p;
        return v;
    }
}

// Streaming variants: the nontemporal hint tells the caches the line is used
// once (a partial read once, a write-back nobody reads again).
__device__ __forceinline__ Vec<16> vload16_stream(const char* p) {
    const u32x4_a4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4_a4*>(p));
    Vec<16> v;
    v.w[0] = x.x; v.w[1] = x.y; v.w[2] = x.z; v.w[3] = x.w;
    return v;
}
__device__ __forceinline__ void vstore16_stream(char* p, const Vec<16>& v) {
    u32x4_a4 x;
    x.x = v.w[0]; x.y = v.w[1]; x.z = v.w[2]; x.w = v.w[3];
    __builtin_nontemporal_store(x, reinterpret_cast<u32x4_a4*>(p));
}
template <int V> __device__ __forceinline__ Vec<V> vload_stream(const char* p) {
    if constexpr (V == 16) return vload16_stream(p); else return vload<V>(p);
}
template <int V> __device__ __forceinline__ void vstore_stream(char* p, const Vec<V>& v) {
    if constexpr (V == 16) vstore16_stream(p, v); else vstore<V>(p, v);
}
// Output stores, streaming or not.  A compile-time choice: the compiler merges
// a runtime branch between the two stores into one plain store.
template <int V, bool NTS> __device__ __forceinline__ void vstore_out(char* p, const Vec<V>& v) {
    if constexpr (NTS) vstore_stream<V>(p, v); else vstore<V>(p, v);
}

__device__ __forceinline__ uint32_t load_word(const char* p) { return *reinterpret_cast<const uint32_t*>(p); }
__device__ __forceinline__ void store_word(char* p, uint32_t w) { *reinterpret_cast<uint32_t*>(p) = w; }
__device__ __forceinline__ float load_f32(const char* p) { return *reinterpret_cast<const float*>(p); }

// --------------------------------------------------------------------------
// payload element types: unpack a vector to fp32 and pack fp32 back with
// round-to-nearest-even.
// --------------------------------------------------------------------------
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf162v __attribute__((ext_vector_type(2)));

struct F32T  { static constexpr int esize = 4; };
struct F16T  { static constexpr int esize = 2; };
struct BF16T { static constexpr int esize = 2; };
struct FP8T  { static constexpr int esize = 1; };   // OCP FP8 E4M3 (e4m3fn)

template <typename DT, int V> struct Cvt;

// 32-bit payload: every word is one element.
template <int V> struct Cvt<F32T, V> {
    static constexpr int n = V / 4;
    static __device__ __forceinline__ void unpack(const Vec<V>& v, float* f) {
#pragma unroll
        for (int k = 0; k < n; ++k) f[k] = __uint_as_float(v.w[k]);
    }
    static __device__ __forceinline__ Vec<V> pack(const float* f) {
        Vec<V> v;
#pragma unroll
        for (int k = 0; k < n; ++k) v.w[k] = __float_as_uint(f[k]);
        return v;
    }
};

// 16-bit payloads, V >= 4: two elements per word, element 2k in the low half.
template <int V> struct Cvt<F16T, V> {
    static constexpr int n = V / 2;
    static __device__ __forceinline__ void unpack(const Vec<V>& v, float* f) {
#pragma unroll
        for (int k = 0; k < V / 4; ++k) {
            half2v h = __builtin_bit_cast(half2v, v.w[k]);
            f[2 * k] = (float)h.x;
            f[2 * k + 1] = (float)h.y;
        }
    }
    static __device__ __forceinline__ Vec<V> pack(const float* f) {
        Vec<V> v;
#pragma unroll
        for (int k = 0; k < V / 4; ++k) {
            half2v h;
            h.x = (_Float16)f[2 * k];
            h.y = (_Float16)f[2 * k + 1];
            v.w[k] = __builtin_bit_cast(uint32_t, h);
        }
        return v;
    }
};
template <> struct Cvt<F16T, 2> {
    static constexpr int n = 1;
    static __device__ __forceinline__ void unpack(const Vec<2>& v, float* f) {
        f[0] = (float)__builtin_bit_cast(_Float16, v.h);
    }
    static __device__ __forceinline__ Vec<2> pack(const float* f) {
        Vec<2> v; v.h = __builtin_bit_cast(uint16_t, (_Float16)f[0]); return v;
    }
};

template <int V> struct Cvt<BF16T, V> {
    static constexpr int n = V / 2;
    static __device__ __forceinline__ void unpack(const Vec<V>& v, float* f) {
#pragma unroll
        for (int k = 0; k < V / 4; ++k) {
            f[2 * k] = __uint_as_float(v.w[k] << 16);
            f[2 * k + 1] = __uint_as_float(v.w[k] & 0xffff0000u);
        }
    }
    static __device__ __forceinline__ Vec<V> pack(const float* f) {
        Vec<V> v;
#pragma unroll
        for (int k = 0; k < V / 4; ++k) {
            bf162v h;
            h.x = (__bf16)f[2 * k];
            h.y = (__bf16)f[2 * k + 1];
            v.w[k] = __builtin_bit_cast(uint32_t, h);
        }
        return v;
    }
};
template <> struct Cvt<BF16T, 2> {
    static constexpr int n = 1;
    static __device__ __forceinline__ void unpack(const Vec<2>& v, float* f) {
        f[0] = __uint_as_float((uint32_t)v.h << 16);
    }
    static __device__ __forceinline__ Vec<2> pack(const float* f) {
        Vec<2> v; v.h = __builtin_bit_cast(uint16_t, (__bf16)f[0]); return v;
    }
};

// 8-bit payload, OCP FP8 E4M3: sign, 4 exponent bits (bias 7), 3 mantissa
// bits; exponent field 0 holds the subnormals m * 2^-9; S.1111.111 is NaN;
// there are no infinities and the largest finite magnitude is 448.
// Decoding and encoding both use gfx950's packed conversions (two values per
// instruction).  The decode is exact.  The hardware encode rounds to nearest
// even but turns magnitudes of 464 and beyond into NaN, so inputs at or
// beyond 448 are first saturated to +-448; with that, the encode below is
// round-to-nearest-even with saturation on every non-NaN fp32 bit pattern
// (tests/fp8_encode_check.hip compares all of them, in both halves of the
// packed word, with a nearest-even reference).  A merged value is a convex combination of fp8
// values and finite (the guards see to that), so the merge never reaches the
// saturation; NaN, which it never forms either, becomes the NaN code 0xff.
__device__ __forceinline__ float fp8_saturate(float f) {
    return fabsf(f) >= 448.0f ? copysignf(448.0f, f) : f;   // NaN fails the test and passes through
}

// Two fp8 codes of a and b into bytes 2*hi and 2*hi + 1 of `word`.
template <bool HI>
__device__ __forceinline__ int fp8_e4m3_pack2(float a, float b, int word) {
    return __builtin_amdgcn_cvt_pk_fp8_f32(fp8_saturate(a), fp8_saturate(b), word, HI);
}

// V >= 4: four elements per word, element 4k in the lowest byte of word k.
template <int V> struct Cvt<FP8T, V> {
    static constexpr int n = V;
    static __device__ __forceinline__ void unpack(const Vec<V>& v, float* f) {
#pragma unroll
        for (int k = 0; k < V / 4; ++k) {
            const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)v.w[k], false);
            const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)v.w[k], true);
            f[4 * k] = lo[0];
            f[4 * k + 1] = lo[1];
            f[4 * k + 2] = hi[0];
            f[4 * k + 3] = hi[1];
        }
    }
    static __device__ __forceinline__ Vec<V> pack(const float* f) {
        Vec<V> v;
#pragma unroll
        for (int k = 0; k < V / 4; ++k)
            v.w[k] = (uint32_t)fp8_e4m3_pack2<true>(f[4 * k + 2], f[4 * k + 3],
                                                    fp8_e4m3_pack2<false>(f[4 * k], f[4 * k + 1], 0));
        return v;
    }
};
template <> struct Cvt<FP8T, 1> {
    static constexpr int n = 1;
    static __device__ __forceinline__ void unpack(const Vec<1>& v, float* f) {
        f[0] = __builtin_amdgcn_cvt_pk_f32_fp8((int)v.b, false)[0];
    }
    static __device__ __forceinline__ Vec<1> pack(const float* f) {
        Vec<1> v; v.b = (uint8_t)(fp8_e4m3_pack2<false>(f[0], 0.0f, 0) & 0xff); return v;
    }
};

// --------------------------------------------------------------------------
// 16-lane DPP rows.  A wave64 is four DPP rows; every reduction below stays
// inside one row and leaves the result in all 16 of its lanes.
// --------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(dpp_i<CTRL>(__float_as_int(v)));
}
// row_ror:n rotates the 16 lanes of each row right by n (DPP controls 0x121-0x12F).
__device__ __forceinline__ float row_max(float v) {
    v = fmaxf(v, dpp_f<0x128>(v));
    v = fmaxf(v, dpp_f<0x124>(v));
    v = fmaxf(v, dpp_f<0x122>(v));
    v = fmaxf(v, dpp_f<0x121>(v));
    return v;
}
__device__ __forceinline__ int row_or(int v) {
    v |= dpp_i<0x128>(v);
    v |= dpp_i<0x124>(v);
    v |= dpp_i<0x122>(v);
    v |= dpp_i<0x121>(v);
    return v;
}
// row_newbcast:i (0x150 + i, gfx90a and later) copies lane i of each row to all its lanes.
template <int I>
__device__ __forceinline__ float row_bcast(float v) { return dpp_f<0x150 + I>(v); }

// Sum over the row.  The rotation tree adds in a different order in every
// lane, so lane 0's total is broadcast to keep the row bit-identical.
__device__ __forceinline__ float row_sum(float v) {
    v += dpp_f<0x128>(v);
    v += dpp_f<0x124>(v);
    v += dpp_f<0x122>(v);
    v += dpp_f<0x121>(v);
    return row_bcast<0>(v);
}

// --------------------------------------------------------------------------
// misc
// --------------------------------------------------------------------------
__device__ __forceinline__ float exp_base(float x, bool base2) { return base2 ? exp2f(x) : expf(x); }
__device__ __forceinline__ float log_base(float x, bool base2) { return base2 ? log2f(x) : logf(x); }
__device__ __forceinline__ bool finite_f(float x) { return __builtin_isfinite(x); }
__device__ __forceinline__ float guard_f(float x) { return __builtin_isfinite(x) ? x : 0.0f; }

// Workgroups are dispatched to the 8 XCDs round-robin (block i runs on XCD
// i mod 8), and each XCD has its own L2.  Renumber blocks so that each XCD
// walks one contiguous range of rows: neighbouring rows share cache lines at
// their ends (interleaved rows are 4-byte aligned), and a line stays in one L2.
__device__ __forceinline__ uint32_t xcd_block() { return xcd_contiguous_order(blockIdx.x, gridDim.x); }

// The same with the XCDs taking turns on chunks of C blocks (block_order.hpp).
template <uint32_t C>
__device__ __forceinline__ uint32_t xcd_chunk_block() { return xcd_chunked_order<C>(blockIdx.x, gridDim.x); }
// ... and computed without a branch on the grid size.
template <uint32_t C>
__device__ __forceinline__ uint32_t xcd_chunk_block_sel() { return xcd_chunked_order_sel<C>(blockIdx.x, gridDim.x); }

__device__ __forceinline__ uint32_t wave_id() {
    return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

}  // namespace dcp
