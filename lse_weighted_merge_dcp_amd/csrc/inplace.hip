// inplace.hip -- the in-place merge of sglang PR #34213 report (code excerpt
// of cp_lse_ag_out_rs_mha): every held partial is overwritten with
// nan_to_num(o) * w, and the merged row is the sum of the scaled partials
// over the ranks, kept for the heads [h0, h1) of this rank's slice.  The page
// does the scaling with PyTorch ops, an all-reduce and a slice copy; here one
// pass reads each partial row once, writes it back once, and writes the slice.
//
// Work mapping: one row group of LPR lanes per (t, h, segment) task, where a
// segment is the LPR x 16 bytes of the row one step of the group covers (a
// 2 KB fp32 row of D = 512 is two segments, two waves).  Each wave then
// issues its loads once and never waits on its own stores (gfx9 counts
// loads and stores in one in-order counter, so a second step would).  Each
// 16-lane DPP row derives G and the weights of all N ranks from the LSE
// stack with DPP reductions (redundantly per segment; it is a few words);
// the payload streams in 16-byte vectors with all P held partials in flight
// per lane, read and written back with the nontemporal hint (each partial
// line is touched once and is dead afterwards).  The fast path (P == N in
// {2,4,8,16}, rank0 == 0: every rank stacked on this GPU) broadcasts weights
// with row_newbcast; otherwise each lane recomputes the weight of the rank
// it streams and applies the guards directly.  In both paths the held rows
// (in the general path, the first block of them and their own LSEs) load
// before the reduction, which does not need them, so a wave's loads share
// one round trip; with a
// single held partial (a rank scaling its own, the call each GPU of a real
// group makes) a task is two consecutive segments of the row, so a wave
// keeps twice the bytes in flight for one reduction.  Guards in the fast path as in
// combine.hip: a finite row sum proves every scaled term finite; otherwise
// the terms are re-formed from guarded values.  Blocks run in plain order
// (measured faster than an XCD-contiguous order for these aligned rows).
#include <math.h>

#include "dcp_device.hpp"
#include "dcp_launch.hpp"

namespace dcp {
namespace {

struct InplK {
    char* part;
    const char* lse;
    char* out;
    char* olse;
    int64_t p_N, p_T, p_H;
    int64_t l_N, l_T, l_H;
    int64_t o_T, o_H;
    int64_t ol_T, ol_H;
    uint32_t rows;  // T * H in this launch
    uint32_t N, P, rank0, H, h0, h1;
    uint32_t chunks, steps;  // steps = segments per row
    FastDiv f_H, f_steps;
    int base2;
};

__device__ __forceinline__ int lse_flags_i(float l) {
    return (__builtin_isnan(l) ? 1 : 0) | (l == INFINITY ? 2 : 0);
}

template <typename DT, int V, int LPR, int NT, int PB, int U, bool NTS>
__global__ __launch_bounds__(256) void inplace_kernel(const InplK k) {
    static_assert(NT == 0 || U == 1, "the stacked-ranks path takes one segment per row group");
    using C = Cvt<DT, V>;
    constexpr int EPV = C::n;
    constexpr uint32_t RPW = 64 / LPR;
    const uint32_t blk = blockIdx.x;
    const uint32_t wave = wave_id();
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t li = lane % LPR;
    const uint32_t g = lane / LPR;
    const uint32_t j = lane & 15u;
    const uint32_t task = (blk * 4u + wave) * RPW + g;
    if (task >= k.rows) return;  // whole row groups leave together
    const bool base2 = k.base2 != 0;

    // a task is U consecutive segments of one row (k.steps tasks per row)
    const uint32_t row = k.steps == 1 ? task : fdiv(task, k.f_steps);
    const uint32_t seg = (task - row * k.steps) * U;
    const uint32_t t = fdiv(row, k.f_H);
    const uint32_t h = row - t * k.H;
    char* pbase = k.part + t * k.p_T + h * k.p_H;
    const char* lbase = k.lse + t * k.l_T + h * k.l_H;
    const bool in_slice = h >= k.h0 && h < k.h1;
    char* obase = (k.out != nullptr && in_slice) ? k.out + t * k.o_T + (h - k.h0) * k.o_H : nullptr;

    // Lanes past the row's last chunk load that chunk again (in bounds) and
    // store nothing.
    bool on[U];
    int64_t coff[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t c = (seg + u) * LPR + li;
        on[u] = c < k.chunks;
        coff[u] = (int64_t)(on[u] ? c : k.chunks - 1u) * V;
    }

    // General path, in blocks of PB held partials: the first block's rows
    // and LSEs do not depend on the reduction below, so they load before it
    // and the wave's loads share one memory round trip.
    Vec<V> x[NT > 0 ? 1 : U][NT > 0 ? 1 : PB];
    float lw[NT > 0 ? 1 : PB];
    if constexpr (NT == 0) {
#pragma unroll
        for (int q = 0; q < PB; ++q) {
            if (q < (int)k.P) {
#pragma unroll
                for (int u = 0; u < U; ++u) x[u][q] = vload_stream<V>(pbase + q * k.p_N + coff[u]);
                lw[q] = load_f32(lbase + (int64_t)(k.rank0 + q) * k.l_N);
            }
        }
    }

    // ---- global LSE over all N ranks -------------------------------------
    const int N = NT > 0 ? NT : (int)k.N;
    float lmax = -INFINITY;
    int fl = 0;
    float lj = -INFINITY;
    // Stacked ranks: all NT partial rows load right after the LSE words,
    // before the reduction that does not need them, so a wave's loads share
    // one memory round trip (measured on MI355X: the Kimi-K3-shaped stacked
    // merge 5.33 -> 5.48 TB/s).
    Vec<V> xs[NT > 0 ? NT : 1];
    if constexpr (NT > 0) {
        if (j < (uint32_t)NT) lj = load_f32(lbase + (int64_t)j * k.l_N);
#pragma unroll
        for (int i = 0; i < NT; ++i) xs[i] = vload_stream<V>(pbase + i * k.p_N + coff[0]);
        fl = lse_flags_i(lj);
        lmax = __builtin_isnan(lj) ? -INFINITY : lj;
    } else {
        for (int i = (int)j; i < N; i += 16) {
            const float l = load_f32(lbase + i * k.l_N);
            fl |= lse_flags_i(l);
            if (!__builtin_isnan(l)) lmax = fmaxf(lmax, l);
        }
    }
    fl = row_or(fl);
    const float m = row_max(lmax);
    float G;
    bool live = false;
    float s = 1.0f;
    if (fl & 1) {
        G = __builtin_nanf("");
    } else if (fl & 2) {
        G = INFINITY;
    } else if (m == -INFINITY) {
        G = -INFINITY;
    } else {
        live = true;
        float part = 0.0f;
        if constexpr (NT > 0) {
            part = (j < (uint32_t)NT) ? exp_base(lj - m, base2) : 0.0f;
        } else {
            for (int i = (int)j; i < N; i += 16) part += exp_base(load_f32(lbase + i * k.l_N) - m, base2);
        }
        s = row_sum(part);
        G = m + log_base(s, base2);
    }

    if constexpr (NT > 0) {
        // ---- fast path: P == N == NT, rank0 == 0 --------------------------
        const float w = (live && j < (uint32_t)NT) ? exp_base(lj - m, base2) / s : 0.0f;
        float wi[NT];
        [&]<int... I>(std::integer_sequence<int, I...>) { ((wi[I] = row_bcast<I>(w)), ...); }
        (std::make_integer_sequence<int, NT>{});
        {
            if (on[0]) {
                const int64_t coff0 = coff[0];
                float sc[NT][EPV];
                float acc[EPV];
#pragma unroll
                for (int e = 0; e < EPV; ++e) acc[e] = 0.0f;
#pragma unroll
                for (int i = 0; i < NT; ++i) {
                    C::unpack(xs[i], sc[i]);
#pragma unroll
                    for (int e = 0; e < EPV; ++e) {
                        sc[i][e] = sc[i][e] * wi[i];
                        acc[e] += sc[i][e];
                    }
                }
                bool bad = false;
#pragma unroll
                for (int e = 0; e < EPV; ++e) bad |= !finite_f(acc[e]);
                if (__builtin_amdgcn_ballot_w64(bad) != 0) {
#pragma unroll
                    for (int e = 0; e < EPV; ++e) acc[e] = 0.0f;
#pragma unroll
                    for (int i = 0; i < NT; ++i) {
                        C::unpack(xs[i], sc[i]);
#pragma unroll
                        for (int e = 0; e < EPV; ++e) {
                            sc[i][e] = guard_f(sc[i][e]) * wi[i];
                            acc[e] += sc[i][e];
                        }
                    }
                }
#pragma unroll
                for (int i = 0; i < NT; ++i) vstore_stream<V>(pbase + i * k.p_N + coff0, C::pack(sc[i]));
                if (obase != nullptr) vstore_out<V, NTS>(obase + coff0, C::pack(acc));
            }
        }
    } else {
        // ---- general path: any N, P held partials starting at rank0 -------
        // (not the stacked-ranks hot path: the guards are applied directly)
        const int P = (int)k.P;
        float acc[U][EPV];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int e = 0; e < EPV; ++e) acc[u][e] = 0.0f;
        for (int j0 = 0; j0 < P; j0 += PB) {
            if (j0 > 0) {
#pragma unroll
                for (int q = 0; q < PB; ++q) {
                    if (j0 + q < P) {
#pragma unroll
                        for (int u = 0; u < U; ++u)
                            x[u][q] = vload_stream<V>(pbase + (j0 + q) * k.p_N + coff[u]);
                        lw[q] = load_f32(lbase + (int64_t)(k.rank0 + j0 + q) * k.l_N);
                    }
                }
            }
            float wv[PB];
#pragma unroll
            for (int q = 0; q < PB; ++q) wv[q] = (live && j0 + q < P) ? exp_base(lw[q] - m, base2) / s : 0.0f;
#pragma unroll
            for (int q = 0; q < PB; ++q) {
                if (j0 + q < P) {
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        float f[EPV];
                        C::unpack(x[u][q], f);
#pragma unroll
                        for (int e = 0; e < EPV; ++e) {
                            f[e] = guard_f(f[e]) * wv[q];
                            acc[u][e] += f[e];
                        }
                        if (on[u]) vstore_stream<V>(pbase + (j0 + q) * k.p_N + coff[u], C::pack(f));
                    }
                }
            }
        }
        if (obase != nullptr) {
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (on[u]) vstore<V>(obase + coff[u], C::pack(acc[u]));
        }
    }
    if (k.olse != nullptr && in_slice && li == 0 && seg == 0)
        *reinterpret_cast<float*>(k.olse + t * k.ol_T + (h - k.h0) * k.ol_H) = G;
}

template <typename DT, int V, int LPR, int NT, int PB = 8, int U = 1, bool NTS = false>
hipError_t run(const InplaceArgs& a, hipStream_t stream) {
    constexpr int64_t RPB = 4 * (64 / LPR);
    const int64_t chunks = a.D * DT::esize / V;
    const int64_t steps = ((chunks + LPR - 1) / LPR + U - 1) / U;  // tasks per row
    const int64_t t_chunk = max_units_per_launch(RPB) / (a.H * steps);
    for (int64_t t0 = 0; t0 < a.T; t0 += t_chunk) {
        const int64_t nt = t0 + t_chunk <= a.T ? t_chunk : a.T - t0;
        InplK k;
        k.part = a.partial + t0 * a.p_T;
        k.lse = a.lse + t0 * a.l_T;
        k.out = a.out ? a.out + t0 * a.o_T : nullptr;
        k.olse = a.out_lse ? a.out_lse + t0 * a.ol_T : nullptr;
        k.p_N = a.p_N; k.p_T = a.p_T; k.p_H = a.p_H;
        k.l_N = a.l_N; k.l_T = a.l_T; k.l_H = a.l_H;
        k.o_T = a.o_T; k.o_H = a.o_H;
        k.ol_T = a.ol_T; k.ol_H = a.ol_H;
        const int64_t rows = nt * a.H * steps;   // (t, h, segment) tasks
        k.rows = (uint32_t)rows;
        k.N = (uint32_t)a.N;
        k.P = (uint32_t)a.P;
        k.rank0 = (uint32_t)a.rank0;
        k.H = (uint32_t)a.H;
        k.h0 = (uint32_t)a.h0;
        k.h1 = (uint32_t)a.h1;
        k.chunks = (uint32_t)chunks;
        k.steps = (uint32_t)steps;
        k.f_H = make_fastdiv(k.H);
        k.f_steps = make_fastdiv(k.steps);
        k.base2 = a.base2 ? 1 : 0;
        const int64_t blocks = (rows + RPB - 1) / RPB;
        const hipError_t e = launch_kernel(inplace_kernel<DT, V, LPR, NT, PB, U, NTS>, dim3((uint32_t)blocks), dim3(256), stream, k, a.timing);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <typename DT, int V, int LPR>
hipError_t run_n(const InplaceArgs& a, hipStream_t stream) {
    if (a.P == a.N && a.rank0 == 0) {
        // a merged slice too large to stay cached for its reader goes out with
        // the nontemporal hint
        if (a.out != nullptr && a.T * (a.h1 - a.h0) * a.D * DT::esize >= kNtOutputBytes) {
            switch (a.N) {
                case 2: return run<DT, V, LPR, 2, 8, 1, true>(a, stream);
                case 4: return run<DT, V, LPR, 4, 8, 1, true>(a, stream);
                case 8: return run<DT, V, LPR, 8, 8, 1, true>(a, stream);
                case 16: return run<DT, V, LPR, 16, 8, 1, true>(a, stream);
                default: break;
            }
        }
        switch (a.N) {
            case 2: return run<DT, V, LPR, 2>(a, stream);
            case 4: return run<DT, V, LPR, 4>(a, stream);
            case 8: return run<DT, V, LPR, 8>(a, stream);
            case 16: return run<DT, V, LPR, 16>(a, stream);
            default: break;
        }
    }
    // one held partial (a rank scaling its own): single-row blocks keep the
    // register budget, and the occupancy, of the smallest case
    if (a.P == 1) return run<DT, V, LPR, 0, 1, 2>(a, stream);
    return run<DT, V, LPR, 0>(a, stream);
}

template <typename DT>
hipError_t run_dt(const InplaceArgs& a, int V, hipStream_t stream) {
    if (V == 16) {
        if constexpr (DT::esize == 1) {
            // fp8 in 8-byte vectors (8 fp32 values per rank and lane): the
            // 16-byte form spills registers with all 16 ranks stacked
            if (a.D / 8 >= 48) return run_n<DT, 8, 64>(a, stream);
            return run_n<DT, 8, 16>(a, stream);
        } else {
            const int64_t chunks = a.D * DT::esize / 16;
            if (chunks >= 48) return run_n<DT, 16, 64>(a, stream);
            return run_n<DT, 16, 16>(a, stream);
        }
    }
    if (a.P == 1) return run<DT, DT::esize, 64, 0, 1, 2>(a, stream);
    return run<DT, DT::esize, 64, 0>(a, stream);
}

}  // namespace

hipError_t launch_inplace(const InplaceArgs& a, hipStream_t stream) {
    if (a.T == 0) return hipSuccess;
    const int esize = dtype_esize(a.dtype);
    int64_t addrs[] = {(int64_t)(uintptr_t)a.partial, a.p_N, a.p_T, a.p_H,
                       (int64_t)(uintptr_t)a.out, a.o_T, a.o_H};
    const int n = a.out ? 7 : 4;
    int V = pick_vec_bytes(a.D * esize, esize, addrs, n);
    if (V != 16) V = esize;
    switch (a.dtype) {
        case DT_F32: return run_dt<F32T>(a, V, stream);
        case DT_F16: return run_dt<F16T>(a, V, stream);
        case DT_FP8: return run_dt<FP8T>(a, V, stream);
        default: return run_dt<BF16T>(a, V, stream);
    }
}

}  // namespace dcp
