// combine.hip -- LSE-weighted merge of N received partials, out of place
// (sglang PR #34651 report, 实现拆解 item 3 receive side; vLLM PR #41160 report,
// 实现拆解 item 1; the nan_to_num guards of sglang PR #34213 report's excerpt).
//
// Per output row (r, b, hl):  G = log_beta sum_i beta^l_i,
// w_i = nan_to_num(beta^(l_i - G)),  out = sum_i w_i * nan_to_num(o_i).
//
// Work mapping.  One row group of LPR lanes (16 or 64) owns one segment
// (LPR x vector bytes) of one output row; rows longer than that are split
// over several groups, each redoing the (tiny) LSE reduction, so no wave
// ever waits on its own stores before loading again.  Inside a group, every
// 16-lane DPP row redundantly derives G and the weights: lane j loads l_j,
// the maximum, the special-value flags and the sum of beta^(l_j - m) are
// reduced with row_ror DPP steps, and each lane's w_j = beta^(l_j - m) / sum
// is broadcast to the row with row_newbcast.  The payload moves in 16-byte
// vectors: every lane loads its chunk of all N peers (N loads in flight) and
// accumulates w_i * o_i in fp32.  Where it pays (short rows, small launches)
// the payload loads go out right after the LSE load, so the reduction
// overlaps them; large launches of long rows load after the weights.
//
// Guards cost nothing on clean data: the sum is formed from the raw values
// and checked once per output element.  A finite sum proves every term was
// finite, i.e. nan_to_num would have changed nothing; otherwise the wave
// reads its rows again and re-forms the sum from the guarded values.
//
// N > 16 (or N not in {2,4,8,16}) takes the general path: lane j handles
// peers j, j+16, ..., and each lane recomputes the weight of each peer as it
// streams (one exp per peer per lane, negligible next to the payload).
#include <math.h>

#include "dcp_device.hpp"
#include "dcp_launch.hpp"

namespace dcp {
namespace {

struct CombK {
    const char* recv;
    const char* rlse;
    char* out;
    char* olse;
    int64_t r_R, r_N, r_B, r_H;
    int64_t rl_R, rl_N, rl_B, rl_H;
    int64_t o_R, o_B, o_H;
    int64_t ol_R, ol_B, ol_H;
    uint32_t rows;    // R * B * Hpr * steps tasks in this launch
    uint32_t N, B, Hpr;
    uint32_t chunks;  // D * esize / V
    uint32_t steps;   // segments per row: ceil(chunks / LPR)
    FastDiv f_Hpr, f_B, f_steps;
    int base2;
};

// Special values and maximum of a row's LSEs, from the l_j (NaN replaced by
// -inf) and flags held by the 16 lanes of each DPP row (lanes past N hold
// -inf).  NaN, +inf or all -inf decide G here and leave live = false (every
// weight 0); otherwise live = true and the caller completes G = m +
// log_beta(s) once it has summed s = sum beta^(l_j - m).
struct LseState {
    float G;
    float m;
    float s;
    bool live;
};

__device__ __forceinline__ LseState reduce_lse(float l_max_in, int flags_in) {
    LseState st;
    const int flags = row_or(flags_in);
    const float m = row_max(l_max_in);
    st.m = m;
    st.s = 0.0f;
    st.live = false;
    if (flags & 1) {
        st.G = __builtin_nanf("");
    } else if (flags & 2) {
        st.G = INFINITY;
    } else if (m == -INFINITY) {
        st.G = -INFINITY;
    } else {
        st.live = true;
        st.G = 0.0f;  // completed by the caller once the sum is known
    }
    return st;
}

__device__ __forceinline__ int lse_flags(float l) {
    return (__builtin_isnan(l) ? 1 : 0) | (l == INFINITY ? 2 : 0);
}

template <typename DT, int V, int LPR, int NT>
__global__ __launch_bounds__(256) void combine_kernel(const CombK k) {
    using C = Cvt<DT, V>;
    constexpr int EPV = C::n;
    constexpr uint32_t RPW = 64 / LPR;
    const uint32_t blk = xcd_block();
    const uint32_t wave = wave_id();
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t li = lane % LPR;
    const uint32_t g = lane / LPR;
    const uint32_t j = lane & 15u;
    const uint32_t task1 = (blk * 4u + wave) * RPW + g;
    // A row group past the end (whole DPP rows) redoes the last task and
    // stores nothing: with no early exit, every argument load goes out before
    // the first wait (one round trip instead of four ahead of the first
    // load; measured on MI355X: the split workload's combine 6.60 -> 6.36 us
    // cold, one destination's 3.60 -> 3.42 us).
    const bool valid = task1 < k.rows;
    const uint32_t task = valid ? task1 : k.rows - 1u;
    const bool base2 = k.base2 != 0;

    const uint32_t row = fdiv(task, k.f_steps);
    const uint32_t seg = task - row * k.steps;
    const uint32_t bb = fdiv(row, k.f_Hpr);
    const uint32_t hl = row - bb * k.Hpr;
    const uint32_t r = fdiv(bb, k.f_B);
    const uint32_t b = bb - r * k.B;
    const char* rbase = k.recv + r * k.r_R + b * k.r_B + hl * k.r_H;
    const char* lbase = k.rlse + r * k.rl_R + b * k.rl_B + hl * k.rl_H;
    char* obase = k.out + r * k.o_R + b * k.o_B + hl * k.o_H;

    if constexpr (NT > 0) {
        // ---- fixed N <= 16: lane j of every DPP row holds peer j ----------
        // The payload loads go out right after the LSE load, so the LSE
        // reduction overlaps them (one memory round trip per wave); lanes
        // past the row end read its last chunk again and never store it.
        float lj = -INFINITY;
        if (j < (uint32_t)NT) lj = load_f32(lbase + (int64_t)j * k.rl_N);
        const uint32_t c = seg * LPR + li;
        const bool on = c < k.chunks;
        const int64_t coff = (int64_t)(on ? c : k.chunks - 1u) * V;
        Vec<V> x[NT];
#pragma unroll
        for (int i = 0; i < NT; ++i) x[i] = vload_stream<V>(rbase + i * k.r_N + coff);
        LseState st = reduce_lse(__builtin_isnan(lj) ? -INFINITY : lj, lse_flags(lj));
        float w = 0.0f;
        if (st.live) {
            const float e = (j < (uint32_t)NT) ? exp_base(lj - st.m, base2) : 0.0f;
            const float s = row_sum(e);
            st.G = st.m + log_base(s, base2);
            w = e / s;
        }
        float wi[NT];
        [&]<int... I>(std::integer_sequence<int, I...>) { ((wi[I] = row_bcast<I>(w)), ...); }
        (std::make_integer_sequence<int, NT>{});

        float acc[EPV];
#pragma unroll
        for (int e = 0; e < EPV; ++e) acc[e] = 0.0f;
#pragma unroll
        for (int i = 0; i < NT; ++i) {
            float f[EPV];
            C::unpack(x[i], f);
#pragma unroll
            for (int e = 0; e < EPV; ++e) acc[e] = fmaf(wi[i], f[e], acc[e]);
        }
        bool bad = false;
#pragma unroll
        for (int e = 0; e < EPV; ++e) bad |= !finite_f(acc[e]);
        if (__builtin_amdgcn_ballot_w64(bad) != 0) {
            // a non-finite payload value: re-form the sum with the guards
#pragma unroll
            for (int e = 0; e < EPV; ++e) acc[e] = 0.0f;
#pragma unroll
            for (int i = 0; i < NT; ++i) {
                float f[EPV];
                C::unpack(vload<V>(rbase + i * k.r_N + coff), f);
#pragma unroll
                for (int e = 0; e < EPV; ++e) acc[e] = fmaf(wi[i], guard_f(f[e]), acc[e]);
            }
        }
        if (on && valid) vstore<V>(obase + coff, C::pack(acc));
        if (k.olse != nullptr && li == 0 && seg == 0 && valid)
            *reinterpret_cast<float*>(k.olse + r * k.ol_R + b * k.ol_B + hl * k.ol_H) = st.G;
    } else {
        // ---- any N: lane j of every DPP row covers peers j, j+16, ... -----
        const int N = (int)k.N;
        float lmax = -INFINITY;
        int fl = 0;
        for (int i = (int)j; i < N; i += 16) {
            const float l = load_f32(lbase + i * k.rl_N);
            fl |= lse_flags(l);
            if (!__builtin_isnan(l)) lmax = fmaxf(lmax, l);
        }
        LseState st = reduce_lse(lmax, fl);
        float s = 1.0f;
        if (st.live) {
            float part = 0.0f;
            for (int i = (int)j; i < N; i += 16) part += exp_base(load_f32(lbase + i * k.rl_N) - st.m, base2);
            s = row_sum(part);
            st.G = st.m + log_base(s, base2);
        }
        constexpr int PB = 8;  // peers in flight per lane
        {
            const uint32_t c = seg * LPR + li;
            if (c < k.chunks) {
                const int64_t coff = (int64_t)c * V;
                float acc[EPV];
#pragma unroll
                for (int e = 0; e < EPV; ++e) acc[e] = 0.0f;
                for (int i0 = 0; i0 < N; i0 += PB) {
                    Vec<V> x[PB];
                    float wv[PB];
#pragma unroll
                    for (int t = 0; t < PB; ++t) {
                        const int i = i0 + t;
                        wv[t] = 0.0f;
                        if (i < N) {
                            x[t] = vload<V>(rbase + i * k.r_N + coff);
                            if (st.live) wv[t] = exp_base(load_f32(lbase + i * k.rl_N) - st.m, base2) / s;
                        }
                    }
#pragma unroll
                    for (int t = 0; t < PB; ++t) {
                        if (i0 + t < N) {
                            float f[EPV];
                            C::unpack(x[t], f);
#pragma unroll
                            for (int e = 0; e < EPV; ++e) acc[e] = fmaf(wv[t], f[e], acc[e]);
                        }
                    }
                }
                bool bad = false;
#pragma unroll
                for (int e = 0; e < EPV; ++e) bad |= !finite_f(acc[e]);
                if (__builtin_amdgcn_ballot_w64(bad) != 0) {
#pragma unroll
                    for (int e = 0; e < EPV; ++e) acc[e] = 0.0f;
                    for (int i = 0; i < N; ++i) {
                        const Vec<V> xv = vload<V>(rbase + i * k.r_N + coff);
                        const float wt = st.live ? exp_base(load_f32(lbase + i * k.rl_N) - st.m, base2) / s : 0.0f;
                        float f[EPV];
                        C::unpack(xv, f);
#pragma unroll
                        for (int e = 0; e < EPV; ++e) acc[e] = fmaf(wt, guard_f(f[e]), acc[e]);
                    }
                }
                if (valid) vstore<V>(obase + coff, C::pack(acc));
            }
        }
        if (k.olse != nullptr && li == 0 && seg == 0 && valid)
            *reinterpret_cast<float*>(k.olse + r * k.ol_R + b * k.ol_B + hl * k.ol_H) = st.G;
    }
}


// Row-per-wave variant (LPR = 64, VB-byte vectors, fixed N <= 16).  The
// row is wave-uniform, so each peer row's base address sits in scalar
// registers and all N loads share one VGPR lane offset; the weights move to
// scalar registers too.  That keeps the kernel at 44 VGPRs for N = 8.  The
// payload is read with the nontemporal hint (each received row is read
// once), which also keeps it from displacing lines the next launch reuses.
//
// HOIST issues the payload loads right after the LSE load, so the LSE
// reduction runs while the payload is in flight: one memory round trip per
// wave instead of two.  That wins when the launch is latency-bound (few
// rows, every wave resident at once) and again on the largest launches;
// in between (thousands of rows, such as one decode layer's combine)
// loading after the weights measured faster, and the launcher picks by
// size.  Small launches
// also use one-wave workgroups (WPB = 1): the rows then spread over up to
// four times as many CUs, and each CU's load pipeline serves fewer of them.
// Block order of the row-per-wave kernel: the XCDs take turns on chunks of
// this many workgroups (1024 rows in 4-wave workgroups).  Grids of at most
// 8 chunks (every launch of up to 2048 workgroups, such as one decode layer
// of the DeepSeek-V3 shape) are XCD-contiguous.  Measured on MI355X against
// the XCD-contiguous order of every launch: long-context B = 512 combine
// (16,384 workgroups) 201 -> 180 us, B = 256 96.4 -> 93.3 us, the
// Kimi-K3-shaped reduce-scatter merge 4.97-5.04 -> 4.85-4.92 ms.  (Chunks of
// 512 gave 176 us at B = 512 but 4.95 ms on the reduce-scatter merge; chunks
// that do not divide a destination's rows, such as 384 or 768 at B = 512,
// were slower than either.)
constexpr uint32_t kWaveChunk = 256;
// Large launches of at most kWaveWideMaxRows rows run in 2-wave workgroups
// whose XCDs take turns on chunks of 1024 of them (2048 rows per chunk; a
// template parameter, like the chunk itself).  Measured on MI355X against
// 4-wave workgroups in chunks of 256: the long-context B = 512 combine
// (65,536 rows) 180 -> 176 us, B = 256 (32,768 rows) 91.4 -> 88.0 us in the
// step (its step +1.1%).  4-wave workgroups in chunks of 1024 and 2048
// (4096 and 8192 rows per turn) took B = 512 to 193 and 201 us.  The
// Kimi-K3-shaped reduce-scatter merge (3.1M rows) keeps 4-wave workgroups
// in chunks of 256, which it prefers.
constexpr uint32_t kWaveChunkWide = 1024;
constexpr int64_t kWaveWideMaxRows = 262144;

// VB = 4 splits each 1 KB segment of the 16-byte form into four, for the
// smallest launches (see kNarrowMaxRows); k.chunks and k.steps then count
// VB-byte vectors.
template <typename DT, int NT, bool HOIST, int WPB, bool NTS, uint32_t CH = kWaveChunk, int VB = 16>
__global__ __launch_bounds__(64 * WPB) void combine_wave_kernel(const CombK k) {
    using C = Cvt<DT, VB>;
    constexpr int EPV = C::n;
    // HOIST launches fetch every argument before their first wait: no branch
    // on the grid size (the selecting form of the block order) or on the row
    // count (a wave past the end redoes task 0 and stores nothing).  Measured
    // on MI355X, two paired runs: one destination's long-context combine at
    // B = 8 2.92 -> 2.76 us, at B = 64 4.62 -> 4.10 us, the B = 8 layer's
    // combine 6.05 -> 5.54 us cold.  The middle range (loads after the
    // weights) keeps the early exit: without it the DeepSeek-V3-shaped
    // combine inside the step went 12.9 -> 13.3 us, its waves' first loads
    // no longer staggered by the argument round trips.
    const uint32_t blk = HOIST ? xcd_chunk_block_sel<CH>() : xcd_chunk_block<CH>();
    const uint32_t wave = wave_id();
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t j = lane & 15u;
    const uint32_t task1 = blk * (uint32_t)WPB + wave;
    if constexpr (!HOIST)
        if (task1 >= k.rows) return;  // wave-uniform
    const bool valid = task1 < k.rows;   // wave-uniform
    const uint32_t task0 = valid ? task1 : k.rows - 1u;
    // Rows run last to first: the combine that follows a pack then starts on
    // the rows whose sends the pack wrote last (measured on MI355X: the
    // DeepSeek-V3-shaped decode step 6.01 -> 6.06 TB/s, its combine 12.1 ->
    // 11.9 us inside the step; cold launches unchanged).
    const uint32_t task = k.rows - 1u - task0;
    const bool base2 = k.base2 != 0;
    const uint32_t row = HOIST ? fdiv(task, k.f_steps) : (k.steps == 1 ? task : fdiv(task, k.f_steps));
    const uint32_t seg = task - row * k.steps;
    const uint32_t bb = fdiv(row, k.f_Hpr);
    const uint32_t hl = row - bb * k.Hpr;
    const uint32_t r = fdiv(bb, k.f_B);
    const uint32_t b = bb - r * k.B;
    const char* rbase = k.recv + r * k.r_R + b * k.r_B + hl * k.r_H;
    const char* lbase = k.rlse + r * k.rl_R + b * k.rl_B + hl * k.rl_H;
    char* obase = k.out + r * k.o_R + b * k.o_B + hl * k.o_H;

    const uint32_t c = seg * 64u + lane;
    const bool on = c < k.chunks;
    // lanes past the row end read its last chunk again (never stored), so
    // the loads need no branch and the LSE wait never covers them
    const uint32_t voff = (on ? c : k.chunks - 1u) * (uint32_t)VB;
    Vec<VB> x[NT];

    float lj = -INFINITY;
    if (j < (uint32_t)NT) lj = load_f32(lbase + (int64_t)j * k.rl_N);
    if constexpr (HOIST) {
#pragma unroll
        for (int i = 0; i < NT; ++i) x[i] = gloadv<VB, true>(wave_addr(rbase + i * k.r_N), voff);
        // keep the loads here: left free, the scheduler sank the 16 loads of
        // the 4-byte form below the wait for the LSE word (one destination's
        // long-context combine at B = 8 3.08 -> 2.96 us); the 16-byte form
        // keeps its own schedule, which the barrier made slower on the
        // largest launches
        if constexpr (VB != 16) __builtin_amdgcn_sched_barrier(0);
    }
    LseState st = reduce_lse(__builtin_isnan(lj) ? -INFINITY : lj, lse_flags(lj));
    float w = 0.0f;
    if (st.live) {
        const float e = (j < (uint32_t)NT) ? exp_base(lj - st.m, base2) : 0.0f;
        const float s = row_sum(e);
        st.G = st.m + log_base(s, base2);
        w = e / s;
    }
    float wi[NT];
    [&]<int... I>(std::integer_sequence<int, I...>) {
        ((wi[I] = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, row_bcast<I>(w))))),
         ...);
    }(std::make_integer_sequence<int, NT>{});
    if constexpr (!HOIST) {
#pragma unroll
        for (int i = 0; i < NT; ++i) x[i] = gloadv<VB, true>(wave_addr(rbase + i * k.r_N), voff);
    }

    float acc[EPV];
#pragma unroll
    for (int e = 0; e < EPV; ++e) acc[e] = 0.0f;
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        float f[EPV];
        C::unpack(x[i], f);
#pragma unroll
        for (int e = 0; e < EPV; ++e) acc[e] = fmaf(wi[i], f[e], acc[e]);
    }
    bool bad = false;
#pragma unroll
    for (int e = 0; e < EPV; ++e) bad |= !finite_f(acc[e]);
    if (__builtin_amdgcn_ballot_w64(bad) != 0) {
        // a non-finite payload value: re-form the sum with the guards (the
        // rows are read again rather than kept live, which would cost VGPRs)
#pragma unroll
        for (int e = 0; e < EPV; ++e) acc[e] = 0.0f;
#pragma unroll
        for (int i = 0; i < NT; ++i) {
            float f[EPV];
            C::unpack(gloadv<VB, false>(wave_addr(rbase + i * k.r_N), voff), f);
#pragma unroll
            for (int e = 0; e < EPV; ++e) acc[e] = fmaf(wi[i], guard_f(f[e]), acc[e]);
        }
    }
    if (on && valid) vstore_out<VB, NTS>(obase + voff, C::pack(acc));
    if (k.olse != nullptr && lane == 0 && seg == 0 && valid)
        *reinterpret_cast<float*>(k.olse + r * k.ol_R + b * k.ol_B + hl * k.ol_H) = st.G;
}

// Launches with at most this many row tasks take the HOIST order (measured
// crossover on MI355X between the latency-bound and the bandwidth-bound
// regime of the row-per-wave kernel).
constexpr int64_t kHoistMaxRows = 2048;
// ... and so do launches of at least this many, in 4-wave workgroups
// (measured on MI355X: the long-context B = 256 combine, 32768 tasks, 96.9 ->
// 95.8 us; the Kimi-K3-shaped reduce-scatter merge 5.05 -> 4.98 ms; the
// DeepSeek-V3-shaped combine, 8192 tasks, 11.9 -> 13.3 us in HOIST order,
// hence the gap).
constexpr int64_t kHoistMinRowsLarge = 32768;
// Launches of at most this many 1 KB row segments run in 4-byte vectors
// (VB = 4): four waves per segment, each converting and summing a quarter
// of the elements.  With so few waves on the chip, a wave's own arithmetic
// (16 peers x 8 elements per lane in the 16-byte form) is not hidden behind
// other waves.  Measured on MI355X, long-context decode (N = 16, D = 512
// bf16), two paired runs: one destination's combine at B = 1 (8 rows) 3.05
// -> 2.70 us, at B = 8 (64 rows) 3.40 -> 3.10 us, the B = 1 layer's
// combine (128 rows) 3.59 -> 3.53 us cold; at 512 rows (B = 64) equal, at
// 1024 (one destination at the DeepSeek-V3 shape) 4.20 -> 4.53 us, and at
// 8-byte vectors nothing gained anywhere.
constexpr int64_t kNarrowMaxRows = 128;

template <typename DT, int V, int LPR, int NT>
hipError_t run(const CombineArgs& a, hipStream_t stream) {
    constexpr int64_t RPB = 4 * (64 / LPR);
    const int64_t chunks = a.D * DT::esize / V;
    const int64_t steps = (chunks + LPR - 1) / LPR;
    const int64_t per_r = a.B * a.Hpr * steps;
    const int64_t lim = max_units_per_launch(RPB);
    int64_t r_chunk = per_r > 0 ? lim / per_r : a.R;
    const bool nt_out = a.R * a.B * a.Hpr * a.D * DT::esize >= kNtOutputBytes;
    int64_t b_chunk = a.B;
    if (r_chunk < 1) {
        r_chunk = 1;
        b_chunk = lim / (a.Hpr * steps);
    }
    for (int64_t r0 = 0; r0 < a.R; r0 += r_chunk) {
        const int64_t nr = r0 + r_chunk <= a.R ? r_chunk : a.R - r0;
        for (int64_t b0 = 0; b0 < a.B; b0 += b_chunk) {
            const int64_t nb = b0 + b_chunk <= a.B ? b_chunk : a.B - b0;
            CombK k;
            k.recv = a.recv + r0 * a.r_R + b0 * a.r_B;
            k.rlse = a.recv_lse + r0 * a.rl_R + b0 * a.rl_B;
            k.out = a.out + r0 * a.o_R + b0 * a.o_B;
            k.olse = a.out_lse ? a.out_lse + r0 * a.ol_R + b0 * a.ol_B : nullptr;
            k.r_R = a.r_R; k.r_N = a.r_N; k.r_B = a.r_B; k.r_H = a.r_H;
            k.rl_R = a.rl_R; k.rl_N = a.rl_N; k.rl_B = a.rl_B; k.rl_H = a.rl_H;
            k.o_R = a.o_R; k.o_B = a.o_B; k.o_H = a.o_H;
            k.ol_R = a.ol_R; k.ol_B = a.ol_B; k.ol_H = a.ol_H;
            const int64_t rows = nr * nb * a.Hpr * steps;   // (r, b, hl, segment) tasks
            k.rows = (uint32_t)rows;
            k.N = (uint32_t)a.N;
            k.B = (uint32_t)nb;
            k.Hpr = (uint32_t)a.Hpr;
            k.chunks = (uint32_t)chunks;
            k.steps = (uint32_t)steps;
            k.f_Hpr = make_fastdiv(k.Hpr);
            k.f_B = make_fastdiv(k.B);
            k.f_steps = make_fastdiv(k.steps);
            k.base2 = a.base2 ? 1 : 0;
            const int64_t blocks = (rows + RPB - 1) / RPB;
            hipError_t e;
            if constexpr (V == 16 && LPR == 64 && NT > 0) {
                if (rows <= kNarrowMaxRows) {
                    // the same tasks in 4-byte vectors: segments of 256 bytes
                    const int64_t ch4 = a.D * DT::esize / 4;
                    const int64_t st4 = (ch4 + 63) / 64;
                    k.chunks = (uint32_t)ch4;
                    k.steps = (uint32_t)st4;
                    k.rows = (uint32_t)(nr * nb * a.Hpr * st4);
                    k.f_steps = make_fastdiv(k.steps);
                    e = launch_kernel(combine_wave_kernel<DT, NT, true, 1, false, kWaveChunk, 4>, dim3(k.rows), dim3(64),
                                      stream, k, a.timing);
                } else if (rows <= kHoistMaxRows)
                    e = launch_kernel(combine_wave_kernel<DT, NT, true, 1, false>, dim3((uint32_t)rows), dim3(64), stream,
                                      k, a.timing);
                else if (rows >= kHoistMinRowsLarge && rows <= kWaveWideMaxRows)
                    e = nt_out ? launch_kernel(combine_wave_kernel<DT, NT, true, 2, true, kWaveChunkWide>,
                                               dim3((uint32_t)((rows + 1) / 2)), dim3(128), stream, k, a.timing)
                               : launch_kernel(combine_wave_kernel<DT, NT, true, 2, false, kWaveChunkWide>,
                                               dim3((uint32_t)((rows + 1) / 2)), dim3(128), stream, k, a.timing);
                else if (rows >= kHoistMinRowsLarge)
                    e = nt_out ? launch_kernel(combine_wave_kernel<DT, NT, true, 4, true>, dim3((uint32_t)blocks),
                                               dim3(256), stream, k, a.timing)
                               : launch_kernel(combine_wave_kernel<DT, NT, true, 4, false>, dim3((uint32_t)blocks),
                                               dim3(256), stream, k, a.timing);
                else if (nt_out)
                    e = launch_kernel(combine_wave_kernel<DT, NT, false, 4, true>, dim3((uint32_t)blocks), dim3(256),
                                      stream, k, a.timing);
                else
                    e = launch_kernel(combine_wave_kernel<DT, NT, false, 4, false>, dim3((uint32_t)blocks), dim3(256),
                                      stream, k, a.timing);
            } else {
                e = launch_kernel(combine_kernel<DT, V, LPR, NT>, dim3((uint32_t)blocks), dim3(256), stream, k, a.timing);
            }
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

template <typename DT, int V, int LPR>
hipError_t run_n(const CombineArgs& a, hipStream_t stream) {
    switch (a.N) {
        case 2: return run<DT, V, LPR, 2>(a, stream);
        case 4: return run<DT, V, LPR, 4>(a, stream);
        case 8: return run<DT, V, LPR, 8>(a, stream);
        case 16: return run<DT, V, LPR, 16>(a, stream);
        default: return run<DT, V, LPR, 0>(a, stream);
    }
}

template <typename DT>
hipError_t run_dt(const CombineArgs& a, int V, hipStream_t stream) {
    if (V == 16) {
        const int64_t chunks = a.D * DT::esize / 16;
        if (chunks >= 48) return run_n<DT, 16, 64>(a, stream);
        // fp8 rows of 384-767 bytes (D = 512: 516-byte interleaved rows):
        // one row per wave in 8-byte vectors rather than 16-lane groups of
        // 16-byte vectors (measured on MI355X: the DeepSeek-V3-shaped fp8
        // combine 10.8 -> 8.9 us inside the step, one destination's 5.2 ->
        // 4.0 us)
        if constexpr (DT::esize == 1)
            if (a.D / 8 >= 48) return run_n<DT, 8, 64>(a, stream);
        return run_n<DT, 16, 16>(a, stream);
    }
    // element-granular fallback for rows that are not 16-byte multiples or
    // not 4-byte aligned
    return run<DT, DT::esize, 64, 0>(a, stream);
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
    if (a.R == 0 || a.B == 0) return hipSuccess;
    const int esize = dtype_esize(a.dtype);
    const int64_t addrs[] = {(int64_t)(uintptr_t)a.recv, a.r_R, a.r_N, a.r_B, a.r_H,
                             (int64_t)(uintptr_t)a.out, a.o_R, a.o_B, a.o_H};
    int V = pick_vec_bytes(a.D * esize, esize, addrs, 9);
    if (V != 16) V = esize;
    switch (a.dtype) {
        case DT_F32: return run_dt<F32T>(a, V, stream);
        case DT_F16: return run_dt<F16T>(a, V, stream);
        case DT_FP8: return run_dt<FP8T>(a, V, stream);
        default: return run_dt<BF16T>(a, V, stream);
    }
}

}  // namespace dcp
