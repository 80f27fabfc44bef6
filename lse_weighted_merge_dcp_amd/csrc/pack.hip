// pack.hip -- stride-driven pack of rank-local partials into per-peer send
// layouts (sglang PR #34651 report, 实现拆解 items 1-3).  The same kernel is
// the strided row copy behind the N == 1 shortcuts of the merge entry points.
//
// Work mapping.  A "row" is one (r, b, h) payload row of row_bytes bytes,
// cut into V-byte chunks.  A row group of LPR lanes (16, 32 or 64) covers
// LPR consecutive chunks of one row per step; rows longer than LPR*V take
// several steps ("virtual rows" = rows x steps).  A 256-thread block runs
// 4 waves x (64/LPR) row groups x U virtual rows, all U loads in flight
// before the U stores, and exits (a one-shot grid: on gfx9 a wave that loops
// waits for its earlier stores before reusing registers, which measured
// slower).  With LPR = 64 a virtual row is wave-uniform, so its index
// arithmetic runs on the scalar unit.  Each payload byte is read once and
// written once; the LSE words of a wave's rows move in one extra load and
// store after the payload.
#include "dcp_device.hpp"
#include "dcp_launch.hpp"

namespace dcp {
namespace {

struct PackK {
    const char* src;
    const char* src_lse;
    char* dst;
    char* dst_lse;
    const char* kv;            // nullable: int32 KV length per (r, b); 0 = neutral row
    int64_t kv_R, kv_B;
    int64_t s_R, s_B, s_H;
    int64_t sl_R, sl_B, sl_H;
    int64_t d_R, d_N, d_B, d_H;
    int64_t dl_R, dl_N, dl_B, dl_H;
    uint32_t vrows;   // rows * steps in this launch
    uint32_t steps;   // ceil(chunks / LPR)
    uint32_t chunks;  // row_bytes / V
    uint32_t H, B, Hpr;
    FastDiv f_steps, f_H, f_B, f_Hpr;
};

constexpr uint32_t kNegInfBits = 0xff800000u;   // -inf as an fp32 word

template <int V, int LPR, int U>
__global__ __launch_bounds__(256) void pack_kernel(const PackK k) {
    static_assert(U <= LPR, "one LSE lane per row of the wave");
    constexpr uint32_t RPW = 64 / LPR;
    // Plain block order: measured faster than an XCD-contiguous renumbering
    // for this pure stream (reads and writes each touch a line once).
    const uint32_t blk = blockIdx.x;
    const uint32_t wave = wave_id();
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t li = lane % LPR;
    const uint32_t g = lane / LPR;

    Vec<V> v[U];
    char* dp[U];
    bool pl[U];
    // The LSE words of the U rows go through lanes li = 0..U-1 of each row
    // group: one load and one store instruction per wave, issued after the
    // payload so they never delay it.
    const char* lsrc = nullptr;
    char* ldst = nullptr;
    // each row's KV length (when given) is read after all payload loads have
    // gone out, so that no payload load waits for it
    const char* kvp[U];
    int lrow = -1;   // which of the U rows the lane's LSE word belongs to
#pragma unroll
    for (int u = 0; u < U; ++u) {
        pl[u] = false;
        kvp[u] = nullptr;
        const uint32_t vrow = (blk * (uint32_t)U + (uint32_t)u) * (4u * RPW) + wave * RPW + g;
        // With several rows per wave, a row group past the end redoes the
        // last row and stores nothing, so no branch stands between the
        // argument loads and the payload loads (measured on MI355X: the split
        // workload's layer 16.3 -> 15.9 us with the same change in the
        // combine).  One-row waves, the smallest launches, keep the early
        // exit, which measured faster there (2-4 workgroups: 1.86 against
        // 1.94 us).
        const bool valid = vrow < k.vrows;
        if (U > 1 || valid) {
            const uint32_t vr = valid ? vrow : k.vrows - 1u;
            const uint32_t row = U > 1 ? fdiv(vr, k.f_steps) : ((k.steps == 1) ? vr : fdiv(vr, k.f_steps));
            const uint32_t step = vr - row * k.steps;
            const uint32_t rb = fdiv(row, k.f_H);
            const uint32_t h = row - rb * k.H;
            const uint32_t r = fdiv(rb, k.f_B);
            const uint32_t b = rb - r * k.B;
            const uint32_t p = fdiv(h, k.f_Hpr);
            const uint32_t hl = h - p * k.Hpr;
            const uint32_t c = step * LPR + li;
            if (k.kv != nullptr && valid) kvp[u] = k.kv + r * k.kv_R + b * k.kv_B;
            if (k.dst != nullptr && c < k.chunks) {
                v[u] = vload<V>(k.src + r * k.s_R + b * k.s_B + h * k.s_H + (int64_t)c * V);
                dp[u] = k.dst + r * k.d_R + p * k.d_N + b * k.d_B + hl * k.d_H + (int64_t)c * V;
                pl[u] = valid;
            }
            if (k.dst_lse != nullptr && valid && step == 0 && li == (uint32_t)u) {
                lsrc = k.src_lse + r * k.sl_R + b * k.sl_B + h * k.sl_H;
                lrow = u;
                ldst = k.dst_lse + r * k.dl_R + p * k.dl_N + b * k.dl_B + hl * k.dl_H;
            }
        }
    }
    uint32_t lw = 0u;
    if (lsrc != nullptr) lw = load_word(lsrc);
    // a token this rank owns no KV for is sent as the neutral pair (zeros and
    // a -inf LSE); its rows were read and are dropped here
    if (k.kv != nullptr) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (kvp[u] != nullptr && load_word(kvp[u]) == 0u) {
                v[u] = vzero<V>();
                if (lrow == u) lw = kNegInfBits;
            }
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
        if (pl[u]) vstore<V>(dp[u], v[u]);
    if (ldst != nullptr) store_word(ldst, lw);
}


// ---------------------------------------------------------------------------
// Interleaved fast path.  In a peer-outer interleaved send buffer the Hpr rows
// of one (rank r, peer p, token b) are one contiguous block of Hpr * W bytes,
// W = row_bytes + 4: each payload row followed by its LSE word.  When that
// block is 16-byte aligned, the pack writes it as a flat stream of aligned
// 16-byte chunks (full-line stores, the LSE words inside them) instead of
// rows that start 4 bytes apart.  The source side of the block is the Hpr
// payload rows of heads p*Hpr.. (contiguous in a [B,H,D] partial), so the
// payload dword j of the block comes from source dword j - k, where k is the
// row it sits in; a chunk that holds the LSE word of row k takes three
// payload dwords from source dwords base-1..base+2 and the LSE in between.
// A wave-step covers 64 chunks (256 dwords).  The lane whose chunk holds
// row k's LSE word loads that word itself, right after its payload load.
// ---------------------------------------------------------------------------
struct StreamK {
    const char* src;
    const char* src_lse;
    char* dst;
    const char* kv;            // nullable: int32 KV length per (r, b); 0 = neutral block
    int64_t kv_R, kv_B;
    int64_t s_R, s_B;          // source bytes per rank / token; head rows are row_bytes apart
    int64_t sl_R, sl_B, sl_H;  // source LSE bytes
    int64_t d_R, d_N, d_B;     // destination block bytes
    uint32_t nsteps;           // R * B * N * S wave-steps in this launch
    uint32_t S;                // wave-steps per block = ceil(Q / 64)
    uint32_t Q;                // 16-byte chunks per block = Hpr * W / 16
    uint32_t Wd;               // dwords per row incl. the LSE word = W / 4 (>= 128)
    uint32_t Hpr, N, B;
    FastDiv f_S, f_N, f_B, f_Wd;
};

// Wave-steps per wave.  One measured fastest on MI355X: 7% faster than two
// on the DeepSeek-V3-shaped pack and up to 20% on small launches, where more
// waves spread the same bytes over more CUs.
constexpr int kStreamU = 1;
// Launches of at least this many wave-steps (and fewer than
// kStreamChunkedSteps, below) use 8-wave workgroups, smaller ones 4-wave
// workgroups, both in plain order (measured: 8-wave 1.5-2% faster at these
// sizes, 1-3% slower on small launches).
constexpr int64_t kStreamWide = 32768;
// Calls whose source partials span at least this many bytes read them with
// the nontemporal hint (each source line is read once).  Above it a layer's
// source and send buffers together outgrow the 256 MB Infinity Cache, and
// keeping the dead source lines out of it leaves the send buffer there for
// whoever reads it next (measured: the long-context B = 64 layer 5.8 ->
// 6.0 TB/s, the combine after the pack 26.5 -> 21.9 us).  Below it the hint
// costs 3% (the DeepSeek-V3-shaped pack, 67 MB of source).
constexpr int64_t kStreamNtSourceBytes = int64_t(96) << 20;

// Calls whose send blocks span at least this many bytes (three times the
// 256 MB Infinity Cache) write them with the nontemporal hint.  Below it
// part of the send buffer is still cached when the combine reads it, and
// that is worth more than faster stores (measured on MI355X, long-context
// decode, 61 layers: B = 512, 1.08 GB of send blocks, step 5,706 -> 5,857
// GB/s, the pack 375 -> 363 us inside the step and 398 -> 362 us cold, the
// combine unchanged; B = 256, 539 MB, step 6,188 -> 5,840 GB/s, its combine
// 95.9 -> 104.6 us; B = 64 -8%).
constexpr int64_t kStreamNtDestBytes = int64_t(768) << 20;

// Launches of at least this many wave-steps run in 4-wave workgroups whose
// XCDs take turns on chunks of kStreamChunk consecutive workgroups (512
// wave-steps a turn) instead of in plain order.  Neighbouring wave-steps
// share the source line at their boundary (the source reads are shifted by
// the LSE words); in one XCD's L2 it is fetched once (the long-context B =
// 512 pack's HBM reads 1.12 -> 1.08 GB).  The order is a template
// parameter: choosing it at run time inside the kernel slowed every launch,
// the small ones most (the fp8 decode pack 14.5 -> 16.1 us).  Measured on
// MI355X, long-context decode, 61 layers, against 8-wave workgroups in plain
// order: B = 64 (147,456 wave-steps) step 6.02 -> 6.49 TB/s, B = 256 6.26 ->
// 6.69, B = 512 6.07 -> 6.21 (with the combine's chunked orders).  8-wave
// workgroups in chunks of 64 gave 1-2% less; chunks of 32, 72 and 128 of
// them within 1% of that, chunks of 256 3% less.  The DeepSeek-V3 pack
// (69,632 wave-steps) lost 2-7% in chunked order (chunks of 8 to 64) and
// keeps the plain one, as do smaller launches.
constexpr uint32_t kStreamChunkedSteps = 131072;
constexpr uint32_t kStreamChunk = 128;

// NTS: send blocks written with the nontemporal hint (a compile-time choice:
// with a runtime flag the compiler merges the two stores into one plain
// store).
//
// No branch stands between the argument loads and the payload load (a wave
// past the end redoes the last wave-step and stores nothing, lanes past a
// block redo its last chunk; the XCD order is computed without a branch),
// and the LSE words are vector loads: scalar loads of data would share the
// out-of-order scalar counter with the argument loads, and a wait on either
// would wait on both.  The argument loads then take one round trip instead of
// two or three before the payload load goes out, which is most of a small
// launch (measured on MI355X, two paired runs: one rank's long-context pack
// at B = 8 2.57 -> 2.31 us, at B = 1 1.96 -> 1.84 us, the DeepSeek-V3 pack
// 24.6 -> 23.8 us cold, the fp8 decode pack 14.5 -> 13.8 us).
//
// SLSE (the middle range of launch sizes, 8-wave workgroups): once the
// payload load has gone out (held there by a scheduling barrier), the
// wave-step's LSE words come through wave-uniform scalar loads instead (the
// first at or after dword d0 belongs to row kl, the next, for rows under
// 1 KB, to row kl + 1).  Measured on MI355X, four paired runs: the
// DeepSeek-V3-shaped step 5,978 -> 6,118 GB/s with them, the fp8 decode step
// 4,828 -> 4,890; on the smallest launches the lanes' own loads stay faster
// (the long-context B = 8 step 3,896 against 3,825), and so do calls with KV
// lengths, whose length load would queue behind the LSE words (the
// DeepSeek-V3 step with them 6,044 against 5,992); the largest launches are
// equal either way.
template <int U, int WPB, bool NTL, bool NTS, uint32_t CH = 0, bool SLSE = false>
__global__ __launch_bounds__(64 * WPB) void pack_stream_kernel(const StreamK k) {
    const uint32_t wave = wave_id();
    const uint32_t lane = threadIdx.x & 63u;
    uint32_t bx = blockIdx.x;
    if constexpr (CH != 0) bx = xcd_chunk_block_sel<CH>();   // XCDs take turns on chunks of CH workgroups
    Vec<16> v[U];
    char* dp[U];
    bool on[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t ws1 = (bx * (uint32_t)U + (uint32_t)u) * (uint32_t)WPB + wave;  // wave-uniform
        const bool valid = ws1 < k.nsteps;
        const uint32_t ws = valid ? ws1 : k.nsteps - 1u;
        const uint32_t blk = fdiv(ws, k.f_S);       // blocks ordered (r, b, p): sequential source reads
        const uint32_t s = ws - blk * k.S;
        const uint32_t rb = fdiv(blk, k.f_N);
        const uint32_t p = blk - rb * k.N;
        const uint32_t r = fdiv(rb, k.f_B);
        const uint32_t b = rb - r * k.B;
        const uint32_t q1 = s * 64u + lane;
        const bool inq = q1 < k.Q;
        const uint32_t q = inq ? q1 : k.Q - 1u;
        const uint32_t j0 = q * 4u;                   // first dword of the chunk
        const uint32_t row = fdiv(j0, k.f_Wd);
        const uint32_t t = k.Wd - 1u - (j0 - row * k.Wd);   // LSE position in the chunk if < 4
        const bool has_lse = t < 4u;
        const uint32_t base = j0 - row;               // source dword of the chunk's first payload dword
        const char* sblk = k.src + r * k.s_R + b * k.s_B + (int64_t)(p * k.Hpr) * ((int64_t)(k.Wd - 1u) * 4);
        const char* sp = sblk + (int64_t)(has_lse ? base - 1u : base) * 4;
        Vec<16> x = NTL ? vload_stream<16>(sp) : vload<16>(sp);
        uint32_t lw = kNegInfBits;
        if constexpr (SLSE) {
            __builtin_amdgcn_sched_barrier(0);
            const uint32_t d0 = s * 256u;
            const uint32_t kl = fdiv(d0, k.f_Wd);
            const uint32_t jl = kl * k.Wd + k.Wd - 1u;
            const char* lrow = k.src_lse + r * k.sl_R + b * k.sl_B + (p * k.Hpr + kl) * k.sl_H;
            uint32_t lval = kNegInfBits, lval1 = kNegInfBits;
            if (kl < k.Hpr && jl >= d0 && jl < d0 + 256u) lval = load_word(lrow);
            if (k.Wd < 256u && kl + 1u < k.Hpr && jl + k.Wd < d0 + 256u) lval1 = load_word(lrow + k.sl_H);
            lw = row != kl ? lval1 : lval;
        } else {
            if (has_lse) lw = load_word(k.src_lse + r * k.sl_R + b * k.sl_B + (p * k.Hpr + row) * k.sl_H);
        }
        // A token this rank owns no KV for is sent as the neutral pair.  Its
        // KV length is read after the payload load has gone out, so the two
        // are in flight together and the block's rows are read (in bounds)
        // and dropped; waiting for the length first cost the
        // DeepSeek-V3-shaped pack 6% (22.2 -> 23.6 us).
        if (k.kv != nullptr) {
            const int kvl = __builtin_nontemporal_load(reinterpret_cast<const int*>(k.kv + r * k.kv_R + b * k.kv_B));
            if (kvl == 0) {
                x = vzero<16>();
                lw = kNegInfBits;
            }
        }
        if (has_lse) {
            uint32_t o[4];
#pragma unroll
            for (int d = 0; d < 4; ++d)
                o[d] = (uint32_t)d < t ? x.w[d + 1] : ((uint32_t)d == t ? lw : x.w[d]);
#pragma unroll
            for (int d = 0; d < 4; ++d) x.w[d] = o[d];
        }
        v[u] = x;
        dp[u] = k.dst + r * k.d_R + p * k.d_N + b * k.d_B + (int64_t)q * 16;
        on[u] = valid && inq;
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
        if (on[u]) vstore_out<16, NTS>(dp[u], v[u]);
}

// True when dst/dst_lse form a peer-outer interleaved buffer whose blocks the
// stream kernel can write: LSE word right after each payload row, rows
// contiguous, 16-byte aligned blocks, rows of at least 512 bytes, and the source
// head rows contiguous and dword aligned.
bool stream_layout(const PackArgs& a) {
    if (a.dst == nullptr || a.dst_lse == nullptr || a.Hpr < 1) return false;
    const int64_t W = a.row_bytes + 4;
    if (a.row_bytes % 4 != 0 || W / 4 < 128) return false;
    if (a.dst_lse != a.dst + a.row_bytes) return false;
    if (a.d_H != W || a.dl_H != W || a.dl_R != a.d_R || a.dl_N != a.d_N || a.dl_B != a.d_B) return false;
    if ((uintptr_t)a.dst % 16 || a.d_R % 16 || a.d_N % 16 || a.d_B % 16 || (a.Hpr * W) % 16) return false;
    if (a.s_H != a.row_bytes || (uintptr_t)a.src % 4 || a.s_R % 4 || a.s_B % 4) return false;
    return true;
}

hipError_t launch_stream(const StreamK& k, bool nt_source, bool nt_dest, hipStream_t stream, CallTiming* t) {
    if (k.nsteps >= kStreamChunkedSteps) {
        const uint32_t blocks = (k.nsteps + 4 * kStreamU - 1) / (4 * kStreamU);
        if (nt_dest)
            return launch_kernel(pack_stream_kernel<kStreamU, 4, true, true, kStreamChunk>, dim3(blocks),
                                 dim3(256), stream, k, t);
        if (nt_source)
            return launch_kernel(pack_stream_kernel<kStreamU, 4, true, false, kStreamChunk>, dim3(blocks),
                                 dim3(256), stream, k, t);
        return launch_kernel(pack_stream_kernel<kStreamU, 4, false, false, kStreamChunk>, dim3(blocks), dim3(256),
                             stream, k, t);
    }
    if (k.nsteps >= kStreamWide) {
        const uint32_t blocks = (k.nsteps + 8 * kStreamU - 1) / (8 * kStreamU);
        if (k.kv == nullptr) {
            if (nt_dest)
                return launch_kernel(pack_stream_kernel<kStreamU, 8, true, true, 0, true>, dim3(blocks), dim3(512),
                                     stream, k, t);
            if (nt_source)
                return launch_kernel(pack_stream_kernel<kStreamU, 8, true, false, 0, true>, dim3(blocks), dim3(512),
                                     stream, k, t);
            return launch_kernel(pack_stream_kernel<kStreamU, 8, false, false, 0, true>, dim3(blocks), dim3(512),
                                 stream, k, t);
        }
        if (nt_dest)
            return launch_kernel(pack_stream_kernel<kStreamU, 8, true, true>, dim3(blocks), dim3(512), stream, k, t);
        if (nt_source)
            return launch_kernel(pack_stream_kernel<kStreamU, 8, true, false>, dim3(blocks), dim3(512), stream, k,
                                 t);
        return launch_kernel(pack_stream_kernel<kStreamU, 8, false, false>, dim3(blocks), dim3(512), stream, k, t);
    }
    const uint32_t blocks = (k.nsteps + 4 * kStreamU - 1) / (4 * kStreamU);
    return launch_kernel(pack_stream_kernel<kStreamU, 4, false, false>, dim3(blocks), dim3(256), stream, k, t);
}

hipError_t run_stream(const PackArgs& a, hipStream_t stream) {
    const int64_t N = a.H / a.Hpr;
    const int64_t W = a.row_bytes + 4;
    const int64_t Q = a.Hpr * W / 16;
    const int64_t S = (Q + 63) / 64;
    const int64_t per_r = a.B * N * S;
    const int64_t lim = max_units_per_launch(4 * kStreamU);
    int64_t r_chunk = lim / per_r;
    int64_t b_chunk = a.B;
    const bool nt_source = a.R * a.B * a.H * a.row_bytes >= kStreamNtSourceBytes;
    const bool nt_dest = a.R * a.B * a.H * W >= kStreamNtDestBytes;
    if (r_chunk < 1) {
        r_chunk = 1;
        b_chunk = lim / (N * S);
    }
    for (int64_t r0 = 0; r0 < a.R; r0 += r_chunk) {
        const int64_t nr = r0 + r_chunk <= a.R ? r_chunk : a.R - r0;
        for (int64_t b0 = 0; b0 < a.B; b0 += b_chunk) {
            const int64_t nb = b0 + b_chunk <= a.B ? b_chunk : a.B - b0;
            StreamK k;
            k.src = a.src + r0 * a.s_R + b0 * a.s_B;
            k.src_lse = a.src_lse + r0 * a.sl_R + b0 * a.sl_B;
            k.dst = a.dst + r0 * a.d_R + b0 * a.d_B;
            k.kv = a.kv ? a.kv + r0 * a.kv_R + b0 * a.kv_B : nullptr;
            k.kv_R = a.kv_R; k.kv_B = a.kv_B;
            k.s_R = a.s_R; k.s_B = a.s_B;
            k.sl_R = a.sl_R; k.sl_B = a.sl_B; k.sl_H = a.sl_H;
            k.d_R = a.d_R; k.d_N = a.d_N; k.d_B = a.d_B;
            k.Q = (uint32_t)Q;
            k.S = (uint32_t)S;
            k.nsteps = (uint32_t)(nr * nb * N * S);
            k.Wd = (uint32_t)(W / 4);
            k.Hpr = (uint32_t)a.Hpr;
            k.N = (uint32_t)N;
            k.B = (uint32_t)nb;
            k.f_S = make_fastdiv(k.S);
            k.f_N = make_fastdiv(k.N);
            k.f_B = make_fastdiv(k.B);
            k.f_Wd = make_fastdiv(k.Wd);
            const hipError_t e = launch_stream(k, nt_source, nt_dest, stream, a.timing);
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

template <int V, int LPR, int U>
hipError_t run_u(const PackArgs& a, hipStream_t stream) {
    constexpr int64_t RPB = 4 * (64 / LPR) * U;
    const int64_t chunks = a.dst ? a.row_bytes / V : 1;
    const int64_t steps = (chunks + LPR - 1) / LPR;
    const int64_t per_r = a.B * a.H * steps;
    // split along R, then along B, so one launch stays within 32-bit indices
    // and grid sizes
    const int64_t lim = max_units_per_launch(RPB);
    int64_t r_chunk = per_r > 0 ? lim / per_r : a.R;
    int64_t b_chunk = a.B;
    if (r_chunk < 1) {
        r_chunk = 1;
        b_chunk = lim / (a.H * steps);
    }
    for (int64_t r0 = 0; r0 < a.R; r0 += r_chunk) {
        const int64_t nr = r0 + r_chunk <= a.R ? r_chunk : a.R - r0;
        for (int64_t b0 = 0; b0 < a.B; b0 += b_chunk) {
            const int64_t nb = b0 + b_chunk <= a.B ? b_chunk : a.B - b0;
            PackK k;
            k.src = a.src ? a.src + r0 * a.s_R + b0 * a.s_B : nullptr;
            k.src_lse = a.src_lse ? a.src_lse + r0 * a.sl_R + b0 * a.sl_B : nullptr;
            k.dst = a.dst ? a.dst + r0 * a.d_R + b0 * a.d_B : nullptr;
            k.dst_lse = a.dst_lse ? a.dst_lse + r0 * a.dl_R + b0 * a.dl_B : nullptr;
            k.kv = a.kv ? a.kv + r0 * a.kv_R + b0 * a.kv_B : nullptr;
            k.kv_R = a.kv_R; k.kv_B = a.kv_B;
            k.s_R = a.s_R; k.s_B = a.s_B; k.s_H = a.s_H;
            k.sl_R = a.sl_R; k.sl_B = a.sl_B; k.sl_H = a.sl_H;
            k.d_R = a.d_R; k.d_N = a.d_N; k.d_B = a.d_B; k.d_H = a.d_H;
            k.dl_R = a.dl_R; k.dl_N = a.dl_N; k.dl_B = a.dl_B; k.dl_H = a.dl_H;
            const int64_t vrows = nr * nb * a.H * steps;
            k.vrows = (uint32_t)vrows;
            k.steps = (uint32_t)steps;
            k.chunks = (uint32_t)chunks;
            k.H = (uint32_t)a.H;
            k.B = (uint32_t)nb;
            k.Hpr = (uint32_t)a.Hpr;
            k.f_steps = make_fastdiv(k.steps);
            k.f_H = make_fastdiv(k.H);
            k.f_B = make_fastdiv(k.B);
            k.f_Hpr = make_fastdiv(k.Hpr);
            const int64_t blocks = (vrows + RPB - 1) / RPB;
            const hipError_t e = launch_kernel(pack_kernel<V, LPR, U>, dim3((uint32_t)blocks), dim3(256), stream, k, a.timing);
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}
// Rows per wave: four when that still leaves at least 512 workgroups, else
// fewer, so small launches spread over more CUs (measured on MI355X: the
// split-layout pack of one rank 5.4 -> 4.5 us with two, the smallest
// interleaved pack 3.4 -> 2.1 us with one).
template <int V, int LPR>
hipError_t run(const PackArgs& a, hipStream_t stream) {
    const int64_t chunks = a.dst ? a.row_bytes / V : 1;
    const int64_t vrows = a.R * a.B * a.H * ((chunks + LPR - 1) / LPR);
    const int64_t per_block = 4 * (64 / LPR);   // rows per workgroup and unit of U
    if (vrows >= 512 * per_block * 4) return run_u<V, LPR, 4>(a, stream);
    if (vrows >= 512 * per_block * 2) return run_u<V, LPR, 2>(a, stream);
    return run_u<V, LPR, 1>(a, stream);
}

template <int V>
hipError_t run_v(const PackArgs& a, hipStream_t stream) {
    const int64_t chunks = a.row_bytes / V;
    if (chunks >= 48) return run<V, 64>(a, stream);
    if (chunks > 16) return run<V, 32>(a, stream);
    return run<V, 16>(a, stream);
}

}  // namespace

int pick_vec_bytes(int64_t row_bytes, int esize, const int64_t* addrs, int count) {
    static const int widths[5] = {16, 8, 4, 2, 1};
    for (int w : widths) {
        if (w < esize) continue;
        if (row_bytes % w != 0) continue;
        const int64_t align = w < 4 ? w : 4;
        bool ok = true;
        for (int i = 0; i < count; ++i) ok = ok && (addrs[i] % align == 0);
        if (ok) return w;
    }
    return esize;
}

hipError_t launch_pack(const PackArgs& a, hipStream_t stream) {
    if (a.R == 0 || a.B == 0) return hipSuccess;
    if (stream_layout(a)) return run_stream(a, stream);
    int V = 4;
    if (a.dst != nullptr) {
        const int64_t addrs[] = {(int64_t)(uintptr_t)a.src, a.s_R, a.s_B, a.s_H,
                                 (int64_t)(uintptr_t)a.dst, a.d_R, a.d_N, a.d_B, a.d_H};
        V = pick_vec_bytes(a.row_bytes, a.esize, addrs, 9);
    }
    switch (V) {
        case 16: return run_v<16>(a, stream);
        case 8: return run_v<8>(a, stream);
        case 4: return run_v<4>(a, stream);
        case 2: return run_v<2>(a, stream);
        default: return run_v<1>(a, stream);
    }
}

}  // namespace dcp
