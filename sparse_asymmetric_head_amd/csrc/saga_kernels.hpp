// saga_kernels.hpp -- HIP kernels for SAGA + Atop-N decode attention on
// gfx950 (CDNA4).  Included once, by saga.hip.
//
// Method ("More Value per Key: Asymmetric Sparse Attention for Faster LLM
// Decoding", picx.dev summary): scores A = q K^T / sqrt(d) over h_k key
// heads (eqs. 2-4); per-element comparison against a per-row threshold tau,
// the row's N-th largest score (Methodology > Atop-N Attention, item 1;
// eq. 6), refreshed exactly every R steps (item 2); softmax over the
// survivors only and a gather-multiply with their value rows from h_v value
// heads (eq. 7; SAGA Architecture).
//
// Kernel map (one decode step):
//   k_select<.., false>  stream K once per key head, MFMA scores for all query
//                        heads of the group, compare with tau, compact the
//                        survivors through LDS into per-(row, segment)
//                        records.                         [HBM-bound, hot]
//   k_attend             per row (d/16 column blocks): read the segment
//                        records, gather the survivors' V rows (the first
//                        fifteen of a segment straight from the record head,
//                        the rest through a wave-local list in LDS), softmax
//                        weights, fp32 accumulation, O.
//   k_attend_row         the same with one block per row, for launches whose
//                        column split would put two blocks or more on a CU.
// Refresh (every R steps) instead runs:
//   k_select<.., true>   same score pass, writes fp32 A
//   k_hist / k_select1 / k_collect / k_select_final   exact radix select
//   k_compact            A >= tau into the same records, then k_attend.
// Dense GQA baseline: k_dense (split-KV online softmax) + k_dense_merge.
//
// Segment records: the survivors of one (row, segment) -- a segment is the
// share of a block's cache positions taken by two of its eight waves, the
// lower wave's list first -- are stored as int32 words
//   [0] count, [1] order key of their largest score, [2+2i] position t_i,
//   [3+2i] bits of score s_i,
// padded to a multiple of 16 words (at least 32), so that the first 128
// bytes hold the count, the key and the first fifteen survivors.
#pragma once

#include "saga_device.hpp"

namespace saga {

#ifndef SAGA_KMAP
#define SAGA_KMAP 1  // k_select: 1 = each MFMA k-step loads contiguous 64-byte half rows
#endif
#ifndef SAGA_SELECT_U
#define SAGA_SELECT_U 1  // k_select: 16-row tiles per wave iteration
#endif
// k_select's tiles per wave iteration on the streaming plan.
template <int D>
constexpr int select_tiles() { return SAGA_SELECT_U; }
#ifndef SAGA_DENSE_U
#define SAGA_DENSE_U 2  // k_dense: 16-row tiles per wave iteration at d = 64 (half at d = 128)
#endif
#ifndef SAGA_KT_LDS
#define SAGA_KT_LDS 1  // k_select: contiguous key loads, moved into the MFMA layout through LDS
#endif
#ifndef SAGA_NT_LOADS
#define SAGA_NT_LOADS 1  // k_select: non-temporal (streaming) loads of the key cache
#endif

constexpr int kWaves = 4;     // waves per workgroup of the streaming kernels; segments per chunk
constexpr int kSelWaves = 2 * kWaves;  // k_select: two waves per segment (two per SIMD)
constexpr int kSelThreads = kSelWaves * kWave;
constexpr int kThreads = kWaves * kWave;
// LDS staging slots per (wave, query head): fewer for groups of more than 32
// query heads, so the staging of eight waves fits the LDS.
template <int NT>
constexpr int cap_w() { return NT > 2 ? 24 : 32; }
constexpr int kMaxSub = 1024; // max segments per row
constexpr int kHistBins = 2048;
constexpr int kHistBlockMax = 8192;  // positions per histogram/collect block
constexpr int kRecHead = 15;  // survivors held in a record's first 128 bytes

// Record order of a chunk's positions.  A chunk of chunk_len positions is
// G = chunk_len / grp groups of grp = 16*U rows (G a multiple of kWaves);
// k_select wave w (of kSelWaves) takes groups w, w + 8, w + 16, ..., and
// waves s and s + 4 share segment s: the segment lists wave s's groups, then
// wave s + 4's.  lo_groups = ceil(G / 8) is the most groups a lower wave
// takes, so the upper wave's list starts at entry lo_groups * grp at most.
__host__ __device__ inline int seg_lo_groups(int chunk_len, int grp) {
    return (chunk_len / grp + kSelWaves - 1) / kSelWaves;
}
// Group (within the chunk) of the k-th group of segment s in record order.
__host__ __device__ inline int seg_group_index(int s, int k, int lo_groups) {
    return k < lo_groups ? s + kSelWaves * k : s + kWaves + kSelWaves * (k - lo_groups);
}

// Rank of cache position t in the order the survivor records list positions
// (a bijection on the positions): chunk; segment s = group % 4; within the
// segment the lower wave's groups, then the upper wave's (above); the
// 16-row tile within the group; inside a tile, output register r = row % 4
// first, then lane quarter row / 4 (the ballot order).
// 32-bit arithmetic: positions, chunk lengths and keys stay below 2^25
// (l_kv * d * 2 < 2^31).
__host__ __device__ inline int record_order_key(int t, int chunk_len, int grp) {
    const int c = t / chunk_len, o = t - c * chunk_len;
    const int gi = o / grp, i = o - gi * grp;
    const int s = gi % kWaves, up = (gi / kWaves) % 2, k = gi / kSelWaves;
    const int q = i % 16;
    return c * chunk_len + s * (chunk_len / kWaves) +
           (up * seg_lo_groups(chunk_len, grp) + k) * grp + (i - q) + (q % 4) * 4 + q / 4;
}

// Words per segment record for a segment capacity of cap survivors.
__host__ __device__ constexpr int64_t seg_words(int64_t cap) {
    return (2 + 2 * cap + 15) / 16 * 16 < 32 ? 32 : (2 + 2 * cap + 15) / 16 * 16;
}

// ------------------------------------------------------------------ select

__device__ __forceinline__ u32x4 ld_k(const void *p) {
#if SAGA_NT_LOADS
    return ld16_stream(p);
#else
    return ld16(p);
#endif
}

struct SelectArgs {
    const uint16_t *Q;   // bf16 [B][h_q][D]
    const uint16_t *K;   // bf16 [B][h_k][l_kv][D]
    const float *tau;    // [B*h_q]            (compare mode)
    float *A;            // [B*h_q][ld_a]      (materialize mode)
    int64_t ld_a;
    int64_t ld_kv;       // rows per key head in K (>= l_kv: a cache with room to grow)
    int B, h_q, h_k;
    int n_chunk;
    int64_t l_kv, chunk_len;
    float scale;
    int32_t *seg;        // [rows][n_sub][seg_w] records
    int n_sub;
    int64_t sub_cap, seg_w;
    uint32_t *hist;      // [rows][kHistBins] radix histograms (materialize mode: cleared here)
    uint32_t *state;     // [rows][4] radix state                (materialize mode: cleared here)
};

// One workgroup = (batch b, key head g, chunk of cache positions), eight
// waves (two per SIMD, so one wave's compare work overlaps the other's
// loads).  Each wave takes groups of U 16-row tiles of K, interleaved across
// the eight waves; waves s and s + 4 share the chunk's segment s.
// MFMA 16x16x32 bf16: A operand = 16 K rows (M = position), B operand = the
// group's query heads (N = head, padded to 16 per N-tile), K dim = d.  At
// k-step s lane l supplies row l%16, d-elements s*32 + (l/16)*8 .. +8, and
// the query operand uses the same permutation of the d axis.  An operand
// register thus holds 16 different rows in every 16-lane quarter, a load
// pattern that costs about 10% of the read bandwidth, so the tiles are
// loaded contiguously (lane l of a load takes 16 bytes at l*16 of a 1 KiB
// run of rows) and moved into the operand layout through a wave-private,
// XOR-swizzled LDS tile (conflict-free 16-byte writes and reads).
// Output: lane l holds rows 4*(l/16)+r, r = 0..3, of query head l%16.
// Survivors are ranked per (wave, head) with ballots (deterministic order:
// tile, then row, then lane), staged in LDS and flushed to the wave's
// segment record of that head.  The record order of the positions is the
// bijection record_order_key below.
template <int D, int NT, bool MATERIALIZE, int U>
__global__ __launch_bounds__(kSelThreads) void k_select(SelectArgs a) {
    // First d-index of the 8 elements lane quarter lq supplies at MFMA
    // k-step s; the query operand uses the same map, so any permutation of
    // the d axis gives the same dot products.
    auto kcol = [](int lq, int s) {
#if SAGA_KMAP
        return s * 32 + lq * 8;          // a k-step reads 64 contiguous bytes of 16 rows
#else
        return lq * (D / 4) + s * 8;     // a lane reads D/2 contiguous bytes of its row
#endif
    };
    constexpr int KS = D / 32;             // MFMA k-steps per row (U: tiles per wave iteration)
    static_assert(U >= 1, "tiles per wave iteration");
    constexpr int QW = D / 4;              // elements of a row per lane quarter
    constexpr int CPR = D / 8;             // 16-byte columns per cache row
    constexpr int RPL = 64 / CPR;          // rows per contiguous wave load
    static_assert(KS * RPL == 16, "a tile is KS contiguous wave loads");
    constexpr int kCapW = cap_w<NT>();
    __shared__ int2 st[MATERIALIZE ? 1 : kSelWaves][MATERIALIZE ? 1 : NT * 16][kCapW];
    __shared__ u32x4 kt[SAGA_KT_LDS ? kSelWaves : 1][SAGA_KT_LDS ? U * 16 * CPR : 1];
    // count and max key of each segment's lower wave, per query head
    __shared__ int2 xlo[MATERIALIZE ? 1 : kWaves][MATERIALIZE ? 1 : NT * 16];

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int ln = lane & 15, lq = lane >> 4;
    const int chunk = blockIdx.x % a.n_chunk;
    const int bg = blockIdx.x / a.n_chunk;
    const int b = bg / a.h_k, g = bg % a.h_k;
    const int j_lo = group_lo(g, a.h_q, a.h_k), j_hi = group_lo(g + 1, a.h_q, a.h_k);
    const int64_t t_begin = (int64_t)chunk * a.chunk_len;
    const int64_t t_end = min(a.l_kv, t_begin + a.chunk_len);
    if constexpr (MATERIALIZE) {
        // The radix select that follows needs zeroed histograms and state for
        // this group's rows (contiguous: rows b*h_q + j_lo .. j_hi); the
        // group's blocks clear them between them, so no earlier call has to
        // leave them at zero.
        const int64_t r0 = (int64_t)b * a.h_q + j_lo, nr = j_hi - j_lo;
        uint32_t *hz = a.hist + r0 * kHistBins, *sz = a.state + r0 * 4;
        const int64_t nthr = blockDim.x;  // four or eight waves
        for (int64_t i = (int64_t)chunk * nthr + threadIdx.x; i < nr * (kHistBins + 4);
             i += (int64_t)a.n_chunk * nthr) {
            if (i < nr * kHistBins) hz[i] = 0u;
            else sz[i - nr * kHistBins] = 0u;
        }
    }

    bf16x8 qop[NT][KS];
    float tau_l[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int j = j_lo + nt * 16 + ln;
        const bool jv = j < j_hi;
        const uint16_t *qp = a.Q + ((int64_t)b * a.h_q + (jv ? j : j_lo)) * D;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            u32x4 r = ld16(qp + kcol(lq, s));
            if (!jv) r = u32x4{0u, 0u, 0u, 0u};
            qop[nt][s] = as_bf16x8(r);
        }
        if (!MATERIALIZE) tau_l[nt] = jv ? a.tau[(int64_t)b * a.h_q + j] : INFINITY;
    }

    int staged[NT], flushed[NT];
    uint32_t mkey[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) staged[nt] = flushed[nt] = 0, mkey[nt] = 0u;

    // segment sw of the chunk; the upper wave (up = 1) lists its survivors
    // after the lower wave's: until the block ends it flushes them from entry
    // ebase = lo_groups * grp (past anything the lower wave can list) and then
    // moves them down to follow the lower wave's count
    const int sw = wave % kWaves, up = wave / kWaves;
    const int sub = chunk * kWaves + sw;
    const int ebase = up ? seg_lo_groups((int)a.chunk_len, 16 * U) * 16 * U : 0;
    const uint64_t head_mask = 0x0001000100010001ull << ln;
    const uint64_t lt_mask = (1ull << lane) - 1ull;
    const uint16_t *Kb = a.K + (int64_t)bg * a.ld_kv * D;

    auto flush = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int j = j_lo + nt * 16 + ln;
            if (j < j_hi) {
                int2 *rec = (int2 *)(a.seg + (((int64_t)b * a.h_q + j) * a.n_sub + sub) * a.seg_w);
                for (int i = lq; i < staged[nt]; i += 4)
                    rec[1 + ebase + flushed[nt] + i] = st[wave][nt * 16 + ln][i];
            }
            flushed[nt] += staged[nt];
            staged[nt] = 0;
        }
    };

    // Score, compare and stage one wave iteration (U tiles starting at t0).
    // INSIDE: the whole iteration lies inside the chunk (every iteration but
    // possibly the last), so the compare needs no position checks.
    auto process = [&](const u32x4 (&kin)[U][KS], int64_t t0, auto inside_tag) __attribute__((always_inline)) {
        constexpr bool INSIDE = decltype(inside_tag)::value;
#if SAGA_KT_LDS
        // Row r, 16-byte column c of tile u sits at slot r*CPR + (c ^ (r & 7)):
        // eight consecutive lanes of either access touch eight distinct bank
        // groups.  The tile is private to the wave, whose LDS accesses run in
        // order, so no barrier is needed.
        u32x4 kr[U][KS];
        u32x4 *w = kt[SAGA_KT_LDS ? wave : 0];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const int r = s * RPL + lane / CPR, c = lane % CPR;
                w[(u * 16 + r) * CPR + (c ^ (r & 7))] = kin[u][s];
            }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const int c = kcol(lq, s) / 8;
                kr[u][s] = w[(u * 16 + ln) * CPR + (c ^ (ln & 7))];
            }
#else
        const u32x4 (&kr)[U][KS] = kin;
#endif
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t tr = t0 + u * 16 + lq * 4;  // position of acc[0]
            const int rem = INSIDE ? 4 : (int)max((int64_t)0, min((int64_t)4, t_end - tr));
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < KS; ++s)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kr[u][s]), qop[nt][s],
                                                                  acc, 0, 0, 0);
                float sc[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) sc[r] = acc[r] * a.scale + 0.0f;  // -0 -> +0
                if (MATERIALIZE) {
                    const int j = j_lo + nt * 16 + ln;
                    if (j < j_hi) {
                        float *Ap = a.A + ((int64_t)b * a.h_q + j) * a.ld_a + tr;
                        if (rem == 4) {
                            *(f32x4 *)Ap = f32x4{sc[0], sc[1], sc[2], sc[3]};
                        } else {
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                if (r < rem) Ap[r] = sc[r];
                        }
                    }
                } else {
                    bool pr[4];
                    uint64_t m[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        pr[r] = INSIDE ? sc[r] >= tau_l[nt] : (r < rem) && (sc[r] >= tau_l[nt]);
                        m[r] = ballot(pr[r]);
                    }
                    if ((m[0] | m[1] | m[2] | m[3]) != 0ull) {
                        int before = 0;
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            if (pr[r]) {
                                const int rank = staged[nt] + before +
                                                 __popcll(m[r] & head_mask & lt_mask);
                                st[wave][nt * 16 + ln][rank] =
                                    int2{(int)(tr + r), __float_as_int(sc[r])};
                                const uint32_t k = fkey(sc[r]);
                                mkey[nt] = mkey[nt] > k ? mkey[nt] : k;
                            }
                            before += __popcll(m[r] & head_mask);
                        }
                        staged[nt] += before;
                    }
                }
            }
            if (!MATERIALIZE) {
                bool full = false;
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) full |= staged[nt] > kCapW - 16;
                if (ballot(full) != 0ull) {
                    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
                    flush();
                }
            }
        }
    };
    // K tiles of one wave iteration.  Rows past the end of the chunk are
    // clamped to its last row (their scores are masked), so the loads need no
    // branches and two buffers can be kept in flight.
    const int64_t last = t_end - 1;
    auto load_tiles = [&](u32x4 (&kr)[U][KS], int64_t t0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
#if SAGA_KT_LDS
#pragma unroll
            for (int s = 0; s < KS; ++s) {   // tile u is KS contiguous 1 KiB wave loads
                int64_t row = t0 + u * 16 + s * RPL + lane / CPR;
                row = row < last ? row : last;
                kr[u][s] = ld_k(Kb + row * D + (lane % CPR) * 8);
            }
#else
            int64_t row = t0 + u * 16 + ln;
            row = row < last ? row : last;
            const uint16_t *kp = Kb + row * D;
#pragma unroll
            for (int s = 0; s < KS; ++s) kr[u][s] = ld_k(kp + kcol(lq, s));
#endif
        }
    };
    constexpr int64_t kStride = kSelWaves * 16 * U;
    int64_t t0 = t_begin + wave * 16 * U;
    if (t0 < t_end) {
        u32x4 ka[U][KS], kb[U][KS];
        // a full iteration, or the chunk's partial last one
        auto step = [&](const u32x4 (&k)[U][KS], int64_t t) __attribute__((always_inline)) {
            if (t + 16 * U <= t_end)
                process(k, t, std::true_type{});
            else
                process(k, t, std::false_type{});
        };
        load_tiles(ka, t0);
        for (;;) {
            load_tiles(kb, t0 + kStride);   // next tiles (clamped past the end)
            step(ka, t0);
            t0 += kStride;
            if (t0 >= t_end) break;
            load_tiles(ka, t0 + kStride);
            step(kb, t0);
            t0 += kStride;
            if (t0 >= t_end) break;
        }
    }
    if constexpr (!MATERIALIZE) {
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        uint32_t mk[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            uint32_t m = mkey[nt];
            uint32_t o = from_xor16(m);
            m = m > o ? m : o;
            o = from_xor32(m);
            mk[nt] = m > o ? m : o;
        }
        // Launched with four waves (chunks of four groups) the lower waves
        // write their records' heads themselves.
        const bool pairs = blockDim.x > kThreads;  // block-uniform
        if (up == 0) {  // wave-uniform: the lower wave's list is final
            flush();
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const int j = j_lo + nt * 16 + ln;
                if (lq == 0 && pairs) xlo[sw][nt * 16 + ln] = int2{flushed[nt], (int)mk[nt]};
                if (lq == 0 && !pairs && j < j_hi) {
                    int2 *rec = (int2 *)(a.seg + (((int64_t)b * a.h_q + j) * a.n_sub + sub) * a.seg_w);
                    rec[0] = int2{flushed[nt], (int)mk[nt]};
                }
            }
        }
        if (!pairs) return;
        __syncthreads();
        if (up == 1) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const int j = j_lo + nt * 16 + ln;
                const int2 lo = xlo[sw][nt * 16 + ln];
                if (j < j_hi) {
                    int2 *rec = (int2 *)(a.seg + (((int64_t)b * a.h_q + j) * a.n_sub + sub) * a.seg_w);
                    // Entries flushed from ebase move down to lo.x (<= ebase):
                    // a round's store lands below every later round's load,
                    // and the store waits for its own round's load.
                    for (int i = lq; i < flushed[nt]; i += 4) {
                        const int2 v = rec[1 + ebase + i];
                        rec[1 + lo.x + i] = v;
                    }
                    for (int i = lq; i < staged[nt]; i += 4)
                        rec[1 + lo.x + flushed[nt] + i] = st[wave][nt * 16 + ln][i];
                    if (lq == 0) {
                        const uint32_t lk = (uint32_t)lo.y;
                        rec[0] = int2{lo.x + flushed[nt] + staged[nt],
                                      (int)(lk > mk[nt] ? lk : mk[nt])};
                    }
                }
            }
        }
    }
}

// ------------------------------------------------------------------ attend

struct AttendArgs {
    const int32_t *seg;  // [rows][n_sub][seg_w] records
    int n_sub;
    int64_t seg_w;
    int sub_cap;         // positions per segment: a record never lists more
    const uint16_t *V;   // bf16 [B][h_v][ld_kv][D], rows < l_kv valid
    int B, h_q, h_v;
    int64_t l_kv, ld_kv;
    float *O;            // [rows][D]
    int32_t *counts;     // [rows] or null
};

constexpr int kAttendWaves = 8;
constexpr int kAttendThreads = kAttendWaves * kWave;
constexpr int kAttendCols = 16;  // output columns per attend block: a lane pair's 2 x 16 bytes
#ifndef SAGA_ATTEND_XCD
#define SAGA_ATTEND_XCD 1  // the blocks of a row share an XCD (and its L2)
#endif
constexpr int kXcds = 8;  // workgroups are dealt round-robin over the 8 XCDs

// Attend blocks per row: block c owns output columns [16c, 16c + 16).
__host__ __device__ constexpr int attend_split(int d) { return d / kAttendCols; }

// Blocks launched for the attend kernel over `rows` rows of head size d.
__host__ __device__ constexpr int64_t attend_grid(int64_t rows, int d) {
    return SAGA_ATTEND_XCD ? (rows + kXcds - 1) / kXcds * kXcds * attend_split(d)
                           : rows * attend_split(d);
}

constexpr int kWaveWin = 256;  // tail survivors staged per wave and window
// Attend launch choices, made per launch by the host (grids of two blocks per
// CU or more take k_attend_row below instead, unless that kernel is compiled
// out):
// DIRECT  survivors per segment gathered straight from the record head: 15
//         (every one the head holds) when one block per CU covers the grid;
//         8 where blocks must share CUs (103 instead of 136 VGPRs, so two
//         8-wave blocks fit on a CU).
// SPREAD  deal a pass's segments round-robin over the eight waves, for rows
//         whose segments average more than fifteen survivors (few, long
//         segments would otherwise leave most waves idle).

// d/16 blocks per row (b, j), block c owning output columns [16c, 16c + 16);
// every block of a row reads the row's records the same way and gathers the
// same survivors in the same lanes and order, so the blocks agree on the
// weight sum and the result is deterministic.
// The two lanes of a pair own one segment of the pass (256 segments per pass
// over the block; pair i of the block, or with SPREAD pair i of wave w
// takes segment 8i + w): each loads one half of the record's first 128
// bytes and they swap halves with DPP, so both hold the count, the max key
// and the first fifteen survivors.  The pair gathers the first DIRECT itself,
// lane h taking columns 8h .. 8h + 8 of the block's sixteen, all loads in
// flight at once, with no list to build first.  Entries past those go
// through a wave-private LDS list (a DPP scan of the tail lengths places
// them; the whole wave loads them, 64 per round) and are gathered by lane
// pairs, 32 per round.  Weights use the wave's running
// maximum (rescaled when a later pass raises it); at the end two block
// barriers give every wave the row maximum, each wave rescales its own sums
// to it, and a thread per column adds the eight waves' sums in a fixed order.
template <int D, int DIRECT, bool SPREAD>
__global__ __launch_bounds__(kAttendThreads) void k_attend(AttendArgs a) {
    constexpr int S = attend_split(D);
    constexpr int EPI = kWave / 2;              // tail survivors per wave round
    constexpr int UN = 4;
    constexpr int SEGP = kAttendThreads / 2;    // segments per pass
    static_assert(S * kAttendCols == D, "attend column split");
    static_assert(DIRECT >= 1 && DIRECT <= kRecHead, "direct survivors come from the record head");
    static_assert(seg_words(1) >= 32, "128-byte record heads");
    __shared__ int wlt[kAttendWaves][kWaveWin];
    __shared__ float wls[kAttendWaves][kWaveWin];
    __shared__ float wpart[kAttendWaves][kAttendCols];
    __shared__ float wlp[kAttendWaves];
    __shared__ float wmx[kAttendWaves];
    __shared__ int wcnt[kAttendWaves];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#if SAGA_ATTEND_XCD
    const int xk = blockIdx.x / kXcds;
    const int csl = xk % S;
    const int row = xk / S * kXcds + blockIdx.x % kXcds;
    if (row >= a.B * a.h_q) return;  // whole block: padding of the last XCD round
#else
    const int row = blockIdx.x / S, csl = blockIdx.x % S;
#endif
    const int32_t *rb = a.seg + (int64_t)row * a.n_sub * a.seg_w;
    const int h = lane & 1;
    // The two lanes of a pair load the halves of their segment's 128-byte head.
    u32x4 own[4];
    // Pair lp of wave w owns segment p0 + 8 lp + w of the pass starting at p0:
    // segments are dealt round-robin over the waves, so rows with few
    // segments still keep every wave busy.
    const int seg_in_pass = SPREAD ? (lane >> 1) * kAttendWaves + wave : tid >> 1;
    auto load_heads = [&](int p0) {
        const int sg = p0 + seg_in_pass;
        const int32_t *rs = rb + (int64_t)sg * a.seg_w;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            own[q] = sg < a.n_sub ? ld16(rs + h * 16 + q * 4) : u32x4{0u, 0u, 0u, 0u};
    };
    load_heads(0);  // first, so the row's setup overlaps the load latency
    const int b = row / a.h_q, j = row % a.h_q;
    const int vh = j * a.h_v / a.h_q;  // j * h_v < 2^30 (h_q <= 32768)
    const uint16_t *Vb = a.V + ((int64_t)b * a.h_v + vh) * a.ld_kv * D + csl * kAttendCols + h * 8;
    int *lt = wlt[wave];
    float *ls = wls[wave];
    const uint32_t lkv_last = (uint32_t)(a.l_kv - 1);  // positions are unsigned-compared with it

    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    float l = 0.f, m_run = -INFINITY;
    int cnt = 0;
    // one gathered half row with weight p (the weight sum counts it on lane 0 of the pair)
    auto add = [&](const u32x4 &v, float p) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc[2 * i] += p * bf_lo(v[i]);
            acc[2 * i + 1] += p * bf_hi(v[i]);
        }
        l += h == 0 ? p : 0.f;
    };
    for (int p0 = 0; p0 < a.n_sub; p0 += SEGP) {
        const int sg = p0 + seg_in_pass;
        if (p0 > 0) load_heads(p0);
        u32x4 hd[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const u32x4 oth = swap_pairs(own[q]);
            hd[q] = h ? oth : own[q];
            hd[4 + q] = h ? own[q] : oth;
        }
        // A record holds at most sub_cap survivors, all inside the cache; a
        // workspace whose last select was for another shape may hold anything,
        // so the count is clamped and positions outside [0, l_kv) are skipped.
        const int n = min(max((int)hd[0][0], 0), a.sub_cap);
        const int nmax = (int)wave_max_u32_dpp((uint32_t)n);  // the wave's longest segment
        if (nmax == 0) continue;  // wave-uniform
        const uint32_t mk = wave_max_u32_dpp(n > 0 ? hd[0][1] : 0u);
        cnt += h == 0 ? n : 0;
        const float m_new = fmaxf(m_run, fkey_inv(mk));
        const float sc = expf(m_run - m_new);  // 0 while m_run is -inf
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] *= sc;
        l *= sc;
        m_run = m_new;
        // The pair's first DIRECT survivors, straight from the registers (past
        // the eighth only when some segment of the wave reaches them: one
        // wave-uniform branch).
        u32x4 vv[DIRECT];
        constexpr int K8 = DIRECT < 8 ? DIRECT : 8;
        // position of head entry k, clamped into the cache for the load; an
        // entry outside it is loaded from the last row and given no weight
        auto tpos = [&](int k) { return hd[(2 + 2 * k) / 4][(2 + 2 * k) % 4]; };
        auto tload = [&](int k) { return (int64_t)min(tpos(k), lkv_last) * D; };
        auto inside = [&](int k) { return tpos(k) <= lkv_last; };
#pragma unroll
        for (int k = 0; k < K8; ++k)
            if (k < n) vv[k] = ld16(Vb + tload(k));
        if (DIRECT > 8 && nmax > 8) {
#pragma unroll
            for (int k = K8; k < DIRECT; ++k)
                if (k < n) vv[k] = ld16(Vb + tload(k));
        }
#pragma unroll
        for (int k = 0; k < K8; ++k)
            if (k < n && inside(k))
                add(vv[k], expf(__uint_as_float(hd[(3 + 2 * k) / 4][(3 + 2 * k) % 4]) - m_run));
        if (DIRECT > 8 && nmax > 8) {
#pragma unroll
            for (int k = K8; k < DIRECT; ++k)
                if (k < n && inside(k))
                    add(vv[k], expf(__uint_as_float(hd[(3 + 2 * k) / 4][(3 + 2 * k) % 4]) - m_run));
        }
        if (nmax <= DIRECT) continue;  // wave-uniform: no tails
        // Tails of the longer segments: entry k >= DIRECT of the pair's segment
        // goes to list slot ex + k - DIRECT.
        const int nt = h == 0 ? max(0, n - DIRECT) : 0;
        const int incl = wave_incl_scan(nt);
        const int tot = __builtin_amdgcn_readlane(incl, 63);
        const int ex = incl - nt;
        const uint64_t big = ballot(nt > 0);
        for (int w0 = 0; w0 < tot; w0 += kWaveWin) {
            const int w1 = min(tot, w0 + kWaveWin);
            for (uint64_t bm = big; bm != 0ull; bm &= bm - 1ull) {
                const int src = __ffsll((unsigned long long)bm) - 1;
                const int sn = __builtin_amdgcn_readlane(n, src);
                const int sx = __builtin_amdgcn_readlane(ex, src) - DIRECT;  // slot of entry k: sx + k
                const int ssg = __builtin_amdgcn_readlane(sg, src);
                const int2 *pr = (const int2 *)(rb + (int64_t)ssg * a.seg_w) + 1;
                const int k0 = max(DIRECT, w0 - sx), k1 = min(sn, w1 - sx);
                for (int k = k0 + lane; k < k1; k += kWave) {
                    const int2 v = pr[k];
                    lt[sx + k - w0] = v.x;
                    ls[sx + k - w0] = __int_as_float(v.y);
                }
            }
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            const int W = w1 - w0;
            for (int e0 = 0; e0 < W; e0 += EPI * UN) {
                int tt[UN];
                float pp[UN];
                u32x4 vt[UN];
#pragma unroll
                for (int u = 0; u < UN; ++u) {
                    const int ei = e0 + u * EPI + (lane >> 1);
                    tt[u] = ei < W ? lt[ei] : -1;
                    pp[u] = ei < W ? ls[ei] : 0.f;
                }
#pragma unroll
                for (int u = 0; u < UN; ++u)
                    vt[u] = (uint32_t)tt[u] <= lkv_last ? ld16(Vb + (int64_t)tt[u] * D)
                                                        : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
                for (int u = 0; u < UN; ++u)
                    if ((uint32_t)tt[u] <= lkv_last) add(vt[u], expf(pp[u] - m_run));
            }
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");  // list reused by the next window
        }
    }
    // Every wave learns the row maximum, rescales its own sums to it in
    // registers and adds its lanes of each column (DPP within 16-lane rows,
    // then the gfx950 row swaps across rows, a fixed order); one thread per column
    // then adds the eight waves' sums in wave order.
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = row_sum_mod<2>(acc[i]);
    l = row_sum_mod<2>(l);
    cnt = __builtin_amdgcn_readlane(wave_incl_scan(cnt), 63);
    if (lane == 0) {
        wmx[wave] = m_run;
        wcnt[wave] = cnt;
    }
    __syncthreads();
    float M = -INFINITY;
#pragma unroll
    for (int q = 0; q < kAttendWaves; ++q) M = fmaxf(M, wmx[q]);
    const float f = cnt > 0 ? expf(m_run - M) : 0.f;  // wave-uniform
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = add_xor32(add_xor16(acc[i] * f));
    l = add_xor32(add_xor16(l * f));
    if (lane < 2) {
#pragma unroll
        for (int i = 0; i < 8; ++i) wpart[wave][h * 8 + i] = acc[i];
        if (h == 0) wlp[wave] = l;
    }
    __syncthreads();
    if (tid < kAttendCols) {
        float so = 0.f, sl = 0.f;
        int total = 0;
#pragma unroll
        for (int q = 0; q < kAttendWaves; ++q) {
            so += wpart[q][tid];
            sl += wlp[q];
            total += wcnt[q];
        }
        a.O[(int64_t)row * D + csl * kAttendCols + tid] = sl > 0.f ? so / sl : 0.f;
        if (tid == 0 && csl == 0 && a.counts) a.counts[row] = total;
    }
}

// Row-per-block attend, for launches whose column split (d/16 blocks per row)
// would put two blocks or more on every compute unit (the host's choice):
// there the column-split blocks run in latency-bound rounds, each re-reading
// the row's records, and a row's whole gather in one block wins (between one
// and two blocks per CU the column split's two dependent round trips, against
// three here, still win on cold caches).  One block of eight waves per row: the segment counts and max keys
// give the row maximum M and, by a block scan, each segment's place in the
// row's list of survivors; windows of kRowWin survivors are then staged in LDS
// (the thread that owns a segment writes its index for each of its entries,
// so every entry is read once, and its weight exp(s - M) computed once), and
// gathered with d/8 lanes per value row, so each load instruction moves whole
// 128- or 256-byte rows, U of them per lane group in flight.  Sums run in a
// fixed order: lanes over their entries, lane groups by DPP and row swaps, waves in
// wave order.  Same clamping of counts and positions as k_attend.
constexpr int kRowWin = 2048;  // survivors staged per window

template <int D>
__global__ __launch_bounds__(kAttendThreads) void k_attend_row(AttendArgs a) {
    constexpr int NW = kAttendWaves;
    constexpr int SPT = kMaxSub / kAttendThreads;  // segments per thread (2)
    constexpr int LPR = D / 8;                     // lanes per value row, 16 bytes each
    constexpr int RPW = kWave / LPR;               // value rows per wave load instruction
    constexpr int U = 8;                           // value-row loads in flight per lane
    constexpr int EPI = NW * RPW * U;              // survivors per block iteration
    static_assert(SPT * kAttendThreads == kMaxSub, "segment split");
    __shared__ int soff[kMaxSub + 1];
    __shared__ uint16_t eseg[kRowWin];
    __shared__ int epos[kRowWin];
    __shared__ float ew[kRowWin];
    __shared__ float wpart[NW][D];
    __shared__ float wl[NW];
    __shared__ uint32_t wmk[NW];
    __shared__ int red[NW];

    const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int32_t *rb = a.seg + (int64_t)row * a.n_sub * a.seg_w;
    // counts (clamped to the segment capacity) and max keys of segments
    // tid * SPT .. tid * SPT + SPT - 1
    int c[SPT], mine = 0;
    uint32_t mk = 0u;
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
        const int sg = tid * SPT + i;
        const int2 hv = sg < a.n_sub ? *(const int2 *)(rb + (int64_t)sg * a.seg_w) : int2{0, 0};
        const int n = min(max(hv.x, 0), a.sub_cap);
        c[i] = n;
        mine += n;
        if (n > 0) mk = mk > (uint32_t)hv.y ? mk : (uint32_t)hv.y;
    }
    const int b = row / a.h_q, j = row % a.h_q;
    const int vh = j * a.h_v / a.h_q;  // j * h_v < 2^30 (h_q <= 32768)
    const int piece = lane % LPR, grp = lane / LPR;
    const uint16_t *Vb = a.V + ((int64_t)b * a.h_v + vh) * a.ld_kv * D + piece * 8;
    const uint32_t lkv_last = (uint32_t)(a.l_kv - 1);  // positions are unsigned-compared with it

    int total;
    const int pre0 = block_excl_scan<NW>(mine, red, &total);
    mk = wave_max_u32_dpp(mk);
    if (lane == 0) wmk[wave] = mk;
    {
        int o = pre0;
#pragma unroll
        for (int i = 0; i < SPT; ++i) {
            const int sg = tid * SPT + i;
            if (sg < a.n_sub) soff[sg] = o;
            o += c[i];
        }
    }
    __syncthreads();
    uint32_t MK = 0u;
#pragma unroll
    for (int w = 0; w < NW; ++w) MK = MK > wmk[w] ? MK : wmk[w];
    const float M = fkey_inv(MK);  // the row maximum (only used when total > 0)

    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    float lsum = 0.f;
    for (int w0 = 0; w0 < total; w0 += kRowWin) {  // block-uniform
        const int W = min(total - w0, kRowWin);
        int o = pre0;
#pragma unroll
        for (int i = 0; i < SPT; ++i) {
            const int k1 = min(o + c[i], w0 + W);
            for (int k = max(o, w0); k < k1; ++k) eseg[k - w0] = (uint16_t)(tid * SPT + i);
            o += c[i];
        }
        __syncthreads();
        // position and weight of every entry of the window; SU loads in flight
        constexpr int SU = 4;
        for (int base = 0; base < W; base += kAttendThreads * SU) {
            int2 v[SU];
#pragma unroll
            for (int u = 0; u < SU; ++u) {
                const int i = min(W - 1, base + u * kAttendThreads + tid);
                const int sg = eseg[i];
                v[u] = ((const int2 *)(rb + (int64_t)sg * a.seg_w))[1 + (w0 + i - soff[sg])];
            }
#pragma unroll
            for (int u = 0; u < SU; ++u) {
                const int i = base + u * kAttendThreads + tid;
                if (i < W) {
                    const bool in = (uint32_t)v[u].x <= lkv_last;
                    const float p = in ? expf(__int_as_float(v[u].y) - M) : 0.f;
                    epos[i] = in ? v[u].x : -1;
                    ew[i] = p;
                    lsum += p;
                }
            }
        }
        __syncthreads();
        for (int e0 = 0; e0 < W; e0 += EPI) {
            int tt[U];
            u32x4 vv[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int e = e0 + (u * NW + wave) * RPW + grp;
                tt[u] = e < W ? epos[e] : -1;
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
                vv[u] = (uint32_t)tt[u] <= lkv_last ? ld16(Vb + (int64_t)tt[u] * D)
                                                    : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if ((uint32_t)tt[u] <= lkv_last) {
                    const float p = ew[e0 + (u * NW + wave) * RPW + grp];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        acc[2 * i] += p * bf_lo(vv[u][i]);
                        acc[2 * i + 1] += p * bf_hi(vv[u][i]);
                    }
                }
            }
        }
        __syncthreads();  // the window's LDS is refilled next
    }
    // lane groups of the wave (same piece), then waves in wave order; each
    // step adds the value of lane l ^ o (add_xor: no LDS but for l ^ 4)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        if constexpr (LPR <= 8) acc[i] = add_xor<8>(acc[i]);
        acc[i] = add_xor<32>(add_xor<16>(acc[i]));
    }
    lsum = add_xor<1>(add_xor<2>(add_xor<4>(add_xor<8>(add_xor<16>(add_xor<32>(lsum))))));
    if (lane < LPR) {
#pragma unroll
        for (int i = 0; i < 8; ++i) wpart[wave][piece * 8 + i] = acc[i];
    }
    if (lane == 0) wl[wave] = lsum;
    __syncthreads();
    if (tid < D) {
        float so = 0.f, sl = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            so += wpart[w][tid];
            sl += wl[w];
        }
        a.O[(int64_t)row * D + tid] = sl > 0.f ? so / sl : 0.f;
        if (tid == 0 && a.counts) a.counts[row] = total;
    }
}

// ------------------------------------------------------------------ refresh

struct RadixArgs {
    const float *A;
    int64_t ld_a, l_kv, N;
    int rows;
    int bpr;          // blocks per row for the histogram/collect passes
    int64_t blk_len;  // positions per block
    uint32_t *hist;   // [rows][2048] (cleared by the materialising score pass)
    uint32_t *state;  // [rows][4]: prefix, rank within bucket, bucket size, fill counter (cleared alike)
    uint32_t *cand;   // [rows][l_kv]
    float *tau;       // [rows]
};

// Digit 1: bits 31..21 of the order key, per-block LDS histogram.  A block
// covers blk_len positions of one row; each thread issues all its float4
// loads before touching the histogram.
constexpr int kRadixVec = kHistBlockMax / (4 * kThreads);  // float4 loads per thread (8)

__device__ __forceinline__ void load_block_scores(const float *Ar, int64_t t0, int64_t t1,
                                                  f32x4 (&v)[kRadixVec]) {
#pragma unroll
    for (int u = 0; u < kRadixVec; ++u) {
        const int64_t t = t0 + ((int64_t)u * kThreads + threadIdx.x) * 4;
        if (t + 3 < t1) {
            v[u] = *(const f32x4 *)(Ar + t);
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c) v[u][c] = (t + c < t1) ? Ar[t + c] : NAN;
        }
    }
}

__global__ __launch_bounds__(kThreads) void k_hist(RadixArgs a) {
    __shared__ uint32_t h[kHistBins];
    const int row = blockIdx.x / a.bpr, blk = blockIdx.x % a.bpr;
    for (int i = threadIdx.x; i < kHistBins; i += kThreads) h[i] = 0u;
    const int64_t t0 = (int64_t)blk * a.blk_len, t1 = min(a.l_kv, t0 + a.blk_len);
    f32x4 v[kRadixVec];
    load_block_scores(a.A + (int64_t)row * a.ld_a, t0, t1, v);
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kRadixVec; ++u)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int64_t t = t0 + ((int64_t)u * kThreads + threadIdx.x) * 4 + c;
            if (t < t1) atomicAdd(&h[fkey(v[u][c]) >> 21], 1u);
        }
    __syncthreads();
    uint32_t *hg = a.hist + (int64_t)row * kHistBins;
    for (int i = threadIdx.x; i < kHistBins; i += kThreads)
        if (h[i]) atomicAdd(hg + i, h[i]);
}

// Scan a histogram from the top bin down; find the bin holding the k-th
// largest element (1-based k).  bins[] in LDS, nbins = 8 * kThreads or less.
__device__ void find_bin_desc(const uint32_t *bins, int nbins, uint32_t k, int *sel_bin,
                              uint32_t *above, int *red) {
    const int per = nbins / kThreads;  // bins per thread (>= 1)
    const int top = nbins - 1 - threadIdx.x * per;
    uint32_t c = 0;
    for (int i = 0; i < per; ++i) c += bins[top - i];
    int total;
    const uint32_t before = (uint32_t)block_excl_scan<kWaves>((int)c, red, &total);
    if (before < k && k <= before + c) {
        uint32_t cum = before;
        for (int i = 0; i < per; ++i) {
            const uint32_t hb = bins[top - i];
            if (cum + hb >= k) {
                *sel_bin = top - i;
                *above = cum;
                break;
            }
            cum += hb;
        }
    }
    __syncthreads();
}

__global__ __launch_bounds__(kThreads) void k_select1(RadixArgs a) {
    __shared__ uint32_t h[kHistBins];
    __shared__ int red[kWaves];
    __shared__ int sel_bin;
    __shared__ uint32_t above;
    const int row = blockIdx.x;
    uint32_t *hg = a.hist + (int64_t)row * kHistBins;
    for (int i = threadIdx.x; i < kHistBins; i += kThreads) h[i] = hg[i];
    if (threadIdx.x == 0) sel_bin = 0, above = 0u;  // (rank N always falls in a bin)
    __syncthreads();
    find_bin_desc(h, kHistBins, (uint32_t)a.N, &sel_bin, &above, red);
    if (threadIdx.x == 0) {
        uint32_t *st = a.state + (int64_t)row * 4;
        st[0] = (uint32_t)sel_bin;
        st[1] = (uint32_t)a.N - above;
        st[2] = h[sel_bin];
    }
}

// Gather the order keys of the bucket holding tau into cand[row]: keys are
// staged in LDS, then one global reservation per block.
__global__ __launch_bounds__(kThreads) void k_collect(RadixArgs a) {
    __shared__ uint32_t keys[kHistBlockMax];
    __shared__ uint32_t nk, base;
    const int row = blockIdx.x / a.bpr, blk = blockIdx.x % a.bpr;
    const uint32_t prefix = a.state[(int64_t)row * 4 + 0];
    uint32_t *fill = a.state + (int64_t)row * 4 + 3;
    const int64_t t0 = (int64_t)blk * a.blk_len, t1 = min(a.l_kv, t0 + a.blk_len);
    if (threadIdx.x == 0) nk = 0u;
    f32x4 v[kRadixVec];
    load_block_scores(a.A + (int64_t)row * a.ld_a, t0, t1, v);
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kRadixVec; ++u)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int64_t t = t0 + ((int64_t)u * kThreads + threadIdx.x) * 4 + c;
            const uint32_t key = fkey(v[u][c]);
            const bool p = t < t1 && (key >> 21) == prefix;
            const uint64_t m = ballot(p);
            if (m) {
                uint32_t wb = 0u;
                if ((threadIdx.x & 63) == 0) wb = atomicAdd(&nk, (uint32_t)__popcll(m));
                wb = __shfl(wb, 0);
                if (p) keys[wb + mbcnt_lt(m)] = key;
            }
        }
    __syncthreads();
    if (threadIdx.x == 0) base = nk ? atomicAdd(fill, nk) : 0u;
    __syncthreads();
    // the row's bucket never holds more than l_kv keys; the clamp only keeps
    // a corrupted fill counter inside the row
    const uint32_t room = base < (uint64_t)a.l_kv ? (uint32_t)(a.l_kv - base) : 0u;
    const uint32_t nw = nk < room ? nk : room;
    uint32_t *cr = a.cand + (int64_t)row * a.l_kv + base;
    for (uint32_t i = threadIdx.x; i < nw; i += kThreads) cr[i] = keys[i];
}

// Finish the select on the bucket's keys: digits 20..10 then 9..0.
__global__ __launch_bounds__(kThreads) void k_select_final(RadixArgs a) {
    __shared__ uint32_t h[kHistBins];
    __shared__ int red[kWaves];
    __shared__ int sel_bin;
    __shared__ uint32_t above;
    const int row = blockIdx.x;
    uint32_t *st = a.state + (int64_t)row * 4;
    const uint32_t prefix = st[0], k = st[1];
    const uint32_t n = st[2] < (uint64_t)a.l_kv ? st[2] : (uint32_t)a.l_kv;  // (never more)
    const uint32_t *cr = a.cand + (int64_t)row * a.l_kv;

    for (int i = threadIdx.x; i < kHistBins; i += kThreads) h[i] = 0u;
    if (threadIdx.x == 0) sel_bin = 0, above = 0u;
    __syncthreads();
    for (uint32_t i = threadIdx.x; i < n; i += kThreads) atomicAdd(&h[(cr[i] >> 10) & 2047u], 1u);
    __syncthreads();
    find_bin_desc(h, kHistBins, k, &sel_bin, &above, red);
    const uint32_t d1 = (uint32_t)sel_bin, k1 = k - above;
    __syncthreads();
    for (int i = threadIdx.x; i < 1024; i += kThreads) h[i] = 0u;
    __syncthreads();
    for (uint32_t i = threadIdx.x; i < n; i += kThreads) {
        const uint32_t key = cr[i];
        if (((key >> 10) & 2047u) == d1) atomicAdd(&h[key & 1023u], 1u);
    }
    __syncthreads();
    find_bin_desc(h, 1024, k1, &sel_bin, &above, red);
    if (threadIdx.x == 0) {
        const uint32_t key = (prefix << 21) | (d1 << 10) | (uint32_t)sel_bin;
        a.tau[row] = fkey_inv(key);
    }
}

// Refresh step selection from the materialised scores: A >= tau into the
// same (row, segment) records k_select writes, in the same record order:
// wave w of the block for (row, chunk) lists segment w, for its record
// indices j = 0, 1, ..., the position whose record_order_key within the
// segment is j.
struct CompactArgs {
    const float *A;
    int64_t ld_a, l_kv, chunk_len, grp;
    int n_chunk;
    const float *tau;
    int32_t *seg;
    int n_sub;
    int64_t sub_cap, seg_w;
};

__global__ __launch_bounds__(kThreads) void k_compact(CompactArgs a) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int row = blockIdx.x / a.n_chunk, chunk = blockIdx.x % a.n_chunk;
    const int sub = chunk * kWaves + wave;
    const int64_t c0 = (int64_t)chunk * a.chunk_len;
    const int64_t t_end = min(a.l_kv, c0 + a.chunk_len);
    const float tau = a.tau[row];
    const float *Ar = a.A + (int64_t)row * a.ld_a;
    int2 *rec = (int2 *)(a.seg + ((int64_t)row * a.n_sub + sub) * a.seg_w);
    const int64_t tiles_per_grp = a.grp / 16;
    const int lo_groups = seg_lo_groups((int)a.chunk_len, (int)a.grp);
    // 16 tiles of the segment per round, in record order; lane l takes tile
    // l / 4, rows 4 * (l % 4) .. +3 (one float4, output registers r = 0..3)
    const int tt = lane >> 2, lq = lane & 3;
    const uint64_t tile_lanes = 0xFull << (4 * tt), below = (1ull << (4 * tt)) - 1ull;
    const uint64_t lt = (1ull << lane) - 1ull;
    int cnt = 0;
    uint32_t mk = 0u;
    const int64_t n_tiles = a.sub_cap / 16;
    for (int64_t T0 = 0; T0 < n_tiles; T0 += 16) {
        const int64_t T = T0 + tt;  // tile of the segment, in record order
        const int64_t k = T / tiles_per_grp, u = T % tiles_per_grp;
        const int64_t t = c0 + (int64_t)seg_group_index(wave, (int)k, lo_groups) * a.grp + u * 16 + lq * 4;
        f32x4 v;
        if (T < n_tiles && t + 3 < t_end) {
            v = *(const f32x4 *)(Ar + t);
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = (T < n_tiles && t + r < t_end) ? Ar[t + r] : -INFINITY;
        }
        bool p[4];
        uint64_t m[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            p[r] = T < n_tiles && t + r < t_end && v[r] >= tau;
            m[r] = ballot(p[r]);
        }
        // rank: survivors of earlier tiles, then of this tile's earlier
        // registers, then of this register's lower lanes
        int rank = cnt;
#pragma unroll
        for (int r = 0; r < 4; ++r) rank += __popcll(m[r] & below);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if (p[r]) {
                rec[1 + rank + __popcll(m[r] & tile_lanes & lt)] =
                    int2{(int)(t + r), __float_as_int(v[r])};
                const uint32_t kv = fkey(v[r]);
                mk = mk > kv ? mk : kv;
            }
            rank += __popcll(m[r] & tile_lanes);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) cnt += __popcll(m[r]);
    }
    mk = wave_max_u32(mk);
    if (lane == 0) rec[0] = int2{cnt, (int)mk};
}

// ------------------------------------------------------------------ refresh from a pivot

// The exact refresh without materialising the scores.  Any N distinct
// positions P give a lower bound on the row's N-th largest score: the least
// of their scores (P is taken as distinct when its record_order_keys
// increase, the order k_refine writes it in).  k_pivot computes it (less a margin that covers the
// difference between its own fp32 sums and the MFMA's), k_select then lists
// every position scoring at least that bound, and k_refine finds the exact
// N-th largest among the listed scores -- they include the N largest -- and
// records N positions of the new survivors as the next refresh's P.

struct PivotArgs {
    const uint16_t *Q, *K;
    int B, h_q, h_k;
    int64_t l_kv, ld_kv, N, chunk_len, grp;
    float scale;
    const int32_t *pivot;  // [rows][N]: positions with increasing record_order_key, else unusable
    float *pi;             // [rows] out: the lower bound (-inf when P is unusable)
};

// Relative margin on |q|.|k| sums: the two fp32 sums of d exact products
// differ by at most 2 (d - 1) 2^-24 of the sum of absolute products, far
// below 2^-12 for d <= 128.
constexpr float kPivotMargin = 1.0f / 4096.0f;

// One block (512 threads) per row; thread i takes pivot positions i, i + 512,
// ...: the position loads, then the key-row loads, all in flight together.
template <int D>
__global__ __launch_bounds__(kAttendThreads) void k_pivot(PivotArgs a) {
    constexpr int NW = kAttendThreads / kWave;
    __shared__ float wmin[NW];
    __shared__ int wbad[NW];
    const int row = blockIdx.x, b = row / a.h_q, j = row % a.h_q;
    const int g = j * a.h_k / a.h_q;  // j * h_k < 2^30 (h_q <= 32768)
    // At d = 64 each thread takes the row's 16-byte parts in its own rotated
    // order, for the query and the key row alike: the addresses then differ
    // across lanes, so the query row comes in vector loads issued with the
    // position loads (at one address for the whole block it was read by two
    // dependent scalar loads before anything else went out).  Any order of the
    // d products is covered by the margin below.  (At d = 128 the rotated
    // vector loads made the kernel slower, 10.3 -> 12.8 us on the Qwen shape;
    // there the row stays at one address.)
    // The positions of a round are loaded a round ahead, the first ones before
    // the query, so the query's loads wait behind nothing.
    const int32_t *P = a.pivot + (int64_t)row * a.N;
    auto positions = [&](int64_t i0, int &p, int &prev) {
        const int64_t i = i0 + threadIdx.x;
        const int64_t ii = i < a.N ? i : a.N - 1;
        p = P[ii];
        prev = ii > 0 ? P[ii - 1] : -1;
    };
    int p_next, prev_next;
    positions(0, p_next, prev_next);
    const int rot = D == 64 ? threadIdx.x % (D / 8) : 0;
    u32x4 qv[D / 8];
#pragma unroll
    for (int c = 0; c < D / 8; ++c) qv[c] = ld16(a.Q + (int64_t)row * D + ((c + rot) % (D / 8)) * 8);
    const uint16_t *Kg = a.K + ((int64_t)b * a.h_k + g) * a.ld_kv * D;
    float mn = INFINITY;
    int bad = 0;
    for (int64_t i0 = 0; i0 < a.N; i0 += kAttendThreads) {
        const int64_t i = i0 + threadIdx.x;
        const int64_t ii = i < a.N ? i : a.N - 1;
        const int p = p_next, prev = prev_next;
        const bool in = p >= 0 && p < a.l_kv;
        // The key row goes out as soon as p is known to be inside the cache;
        // a pivot that fails the order check makes the bound -inf anyway.
        const uint16_t *kr = Kg + (int64_t)(in ? p : 0) * D;
        u32x4 kv[D / 8];
#pragma unroll
        for (int c = 0; c < D / 8; ++c) kv[c] = ld16(kr + ((c + rot) % (D / 8)) * 8);
        if (i0 + kAttendThreads < a.N) positions(i0 + kAttendThreads, p_next, prev_next);
        const int cl = (int)a.chunk_len, gp = (int)a.grp;
        const int kp = in ? record_order_key(p, cl, gp) : -1;
        const int kq = ii == 0 ? -1
                     : (prev >= 0 && prev < a.l_kv ? record_order_key(prev, cl, gp) : INT32_MAX);
        const bool ok = in && kp > kq;  // inside the cache, distinct (increasing keys)
        if (i < a.N) bad |= !ok;
        float s = 0.f, e = 0.f;
#pragma unroll
        for (int c = 0; c < D / 8; ++c)
#pragma unroll
            for (int i2 = 0; i2 < 4; ++i2) {
                const float p0 = bf_lo(qv[c][i2]) * bf_lo(kv[c][i2]);
                const float p1 = bf_hi(qv[c][i2]) * bf_hi(kv[c][i2]);
                s += p0 + p1;
                e += fabsf(p0) + fabsf(p1);
            }
        const float sc = s * a.scale - (e * a.scale * kPivotMargin + 1e-30f);
        if (i < a.N) mn = fminf(mn, sc);
    }
    mn = fkey_inv(~wave_max_u32_dpp(~fkey(mn)));  // the wave's least (keys order as the floats)
    bad = ballot(bad != 0) != 0ull;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) {
        wmin[wave] = mn;
        wbad[wave] = bad;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        float m = INFINITY;
        int bd = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            m = fminf(m, wmin[w]);
            bd += wbad[w];
        }
        a.pi[row] = bd ? -INFINITY : m;
    }
}

struct RefineArgs {
    int32_t *seg;        // [rows][n_sub][seg_w] records of every score >= pi; rewritten to S
    int n_sub;
    int64_t seg_w, sub_cap, N;
    float *tau;          // [rows] out: the exact N-th largest score
    int32_t *pivot;      // [rows][N] out: positions of N survivors, in record order
};

constexpr int kRefineCap = 5120;  // listed scores staged in LDS (two blocks fit a CU)

// One block per row.  The listed scores (up to kRefineCap staged in LDS with
// their positions and segments; more than that first go through one radix
// digit read from the records, and only the keys at or above the lower edge
// of the bucket holding rank N are staged; if even those are too many, the
// records are read on every pass) go through radix digits of their order
// keys, from the highest bit in which they differ, until the bucket holding
// rank N is small enough to rank its keys against each other directly; that
// gives the exact key of rank N.
// The survivors (score >= tau) are then walked in record
// order: the first N positions go to pivot, and every record is rewritten in
// place to its survivors (same order; the max key stays right, since a record
// that keeps any survivor keeps its largest).
__global__ __launch_bounds__(kThreads) void k_refine(RefineArgs a) {
    constexpr int SPT = kMaxSub / kThreads;  // segments per thread (4)
    constexpr int SU = 8;                    // staging loads in flight per thread
    __shared__ uint32_t ekey[kRefineCap];
    __shared__ int epos[kRefineCap];
    __shared__ uint16_t eseg[kRefineCap];
    __shared__ uint32_t h[kHistBins];
    __shared__ int soff[kMaxSub + 1];
    __shared__ int pcnt[kMaxSub], pbase[kMaxSub];
    __shared__ int red[kWaves];
    __shared__ int sel_bin;
    __shared__ uint32_t above;
    __shared__ uint32_t cand[kThreads];
    __shared__ int ncand;
    __shared__ uint32_t sel_key;
    __shared__ uint32_t rmn[kWaves], rmx[kWaves];
    const int row = blockIdx.x, tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    int32_t *rb = a.seg + (int64_t)row * a.n_sub * a.seg_w;

    int total = 0;
    bool staged = false;
    uint32_t kmn = 0xffffffffu, kmx = 0u;  // least and largest listed key
    // segment of flattened entry i (soff is non-decreasing)
    auto seg_of = [&](int i) {
        int lo = 0, hi = a.n_sub - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (soff[mid] <= i) lo = mid;
            else hi = mid - 1;
        }
        return lo;
    };
    auto entry_ptr = [&](int sgi, int i) {
        return (const int2 *)(rb + (int64_t)sgi * a.seg_w) + 1 + (i - soff[sgi]);
    };

    // Rows of at most kThreads segments whose listing fits the LDS: a thread
    // per segment reads the record head (count, max key, first kRecHead
    // entries) in one 128-byte read, the block scan places the segment, and
    // the thread stages its entries (reading any past the head, SU at a time)
    // with their keys' least and largest value -- one read round instead of
    // counts, then entries, then a pass for the key range.
    bool fast = false;
    int f_off = 0, f_n = 0;  // fast: this thread's segment's entries in the staged list
    if (a.n_sub <= kThreads) {  // block-uniform
        const int sgi = tid;
        u32x4 hd[8];
#pragma unroll
        for (int q = 0; q < 8; ++q)
            hd[q] = sgi < a.n_sub ? ld16(rb + (int64_t)sgi * a.seg_w + q * 4) : u32x4{0u, 0u, 0u, 0u};
        const int n = min(max((int)hd[0][0], 0), (int)a.sub_cap);
        const int o = block_excl_scan<kWaves>(n, red, &total);
        if (total > 0 && total <= kRefineCap) {  // block-uniform
            fast = staged = true;
            f_off = o, f_n = n;
            uint32_t mn = 0xffffffffu, mx = 0u;
#pragma unroll
            for (int k = 0; k < kRecHead; ++k)
                if (k < n) {
                    const uint32_t key = fkey(__uint_as_float(hd[(3 + 2 * k) / 4][(3 + 2 * k) % 4]));
                    epos[o + k] = (int)hd[(2 + 2 * k) / 4][(2 + 2 * k) % 4];
                    ekey[o + k] = key;
                    eseg[o + k] = (uint16_t)sgi;
                    mn = mn < key ? mn : key;
                    mx = mx > key ? mx : key;
                }
            const int2 *es = (const int2 *)(rb + (int64_t)sgi * a.seg_w) + 1;
            for (int k0 = kRecHead; k0 < n; k0 += SU) {
                int2 v[SU];
#pragma unroll
                for (int u = 0; u < SU; ++u) v[u] = es[min(n - 1, k0 + u)];
#pragma unroll
                for (int u = 0; u < SU; ++u)
                    if (k0 + u < n) {
                        const uint32_t key = fkey(__int_as_float(v[u].y));
                        epos[o + k0 + u] = v[u].x;
                        ekey[o + k0 + u] = key;
                        eseg[o + k0 + u] = (uint16_t)sgi;
                        mn = mn < key ? mn : key;
                        mx = mx > key ? mx : key;
                    }
            }
            if (sgi < a.n_sub) {
                soff[sgi] = o;
                pcnt[sgi] = 0;
            }
            if (tid == 0) {
                soff[a.n_sub] = total;
                sel_bin = 0;
                above = 0u;
                ncand = 0;
            }
            mn = ~wave_max_u32_dpp(~mn);
            mx = wave_max_u32_dpp(mx);
            if (lane == 0) {
                rmn[wave] = mn;
                rmx[wave] = mx;
            }
            __syncthreads();
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                kmn = kmn < rmn[w] ? kmn : rmn[w];
                kmx = kmx > rmx[w] ? kmx : rmx[w];
            }
        }
    }
    // fn(i, key) for the listed entries i = i0, i0 + di, ... below i1; from the
    // records (too many to stage) SU loads go out together before any is used
    auto for_keys = [&](int i0, int i1, int di, auto &&fn) __attribute__((always_inline)) {
        if (staged) {
            for (int i = i0; i < i1; i += di) fn(i, ekey[i]);
            return;
        }
        for (int base = i0; base < i1; base += di * SU) {
            uint32_t k[SU];
#pragma unroll
            for (int u = 0; u < SU; ++u) {
                const int i = min(i1 - 1, base + u * di);
                k[u] = fkey(__int_as_float(entry_ptr(seg_of(i), i)->y));
            }
#pragma unroll
            for (int u = 0; u < SU; ++u)
                if (base + u * di < i1) fn(base + u * di, k[u]);
        }
    };

    if (!fast) {
        // segment counts -> offsets of the flattened list
        int c[SPT], mine = 0;
#pragma unroll
        for (int i = 0; i < SPT; ++i) {
            const int sgi = tid * SPT + i;
            int n = sgi < a.n_sub ? rb[(int64_t)sgi * a.seg_w] : 0;
            n = n < 0 ? 0 : (n > a.sub_cap ? (int)a.sub_cap : n);
            c[i] = n;
            mine += n;
        }
        const int pre0 = block_excl_scan<kWaves>(mine, red, &total);
        int pre = pre0;
#pragma unroll
        for (int i = 0; i < SPT; ++i) {
            const int sgi = tid * SPT + i;
            if (sgi < a.n_sub) {
                soff[sgi] = pre;
                pcnt[sgi] = 0;
            }
            pre += c[i];
        }
        if (tid == 0) {
            soff[a.n_sub] = total;
            sel_bin = 0;
            above = 0u;
            ncand = 0;
        }
        __syncthreads();
        if (total == 0) return;  // block-uniform; no survivors listed (cannot happen for N >= 1)
        staged = total <= kRefineCap;
        if (staged) {
            // the segment of every flattened entry, written by the thread that
            // owns the segment, so each staging load needs one LDS read
            int o = pre0;
#pragma unroll
            for (int i = 0; i < SPT; ++i) {
                for (int k = 0; k < c[i]; ++k) eseg[o + k] = (uint16_t)(tid * SPT + i);
                o += c[i];
            }
            __syncthreads();
            for (int base = 0; base < total; base += kThreads * SU) {
                int2 v[SU];
#pragma unroll
                for (int u = 0; u < SU; ++u) {
                    const int i = min(total - 1, base + u * kThreads + tid);
                    v[u] = *entry_ptr(eseg[i], i);
                }
#pragma unroll
                for (int u = 0; u < SU; ++u) {
                    const int i = base + u * kThreads + tid;
                    if (i < total) {
                        epos[i] = v[u].x;
                        ekey[i] = fkey(__int_as_float(v[u].y));
                    }
                }
            }
            __syncthreads();
        }
        if (!staged) {
            // Too many listed to stage: one radix digit over the records finds
            // the bucket that holds rank N; the keys at or above its lower edge
            // (every key above tau among them) are staged in record order and
            // the rest of the search runs on them.
            uint32_t fmn = 0xffffffffu, fmx = 0u;
            for_keys(tid, total, kThreads, [&](int, uint32_t k) {
                fmn = fmn < k ? fmn : k;
                fmx = fmx > k ? fmx : k;
            });
            fmn = ~wave_max_u32_dpp(~fmn);
            fmx = wave_max_u32_dpp(fmx);
            if (lane == 0) {
                rmn[wave] = fmn;
                rmx[wave] = fmx;
            }
            for (int i = tid; i < kHistBins; i += kThreads) h[i] = 0u;
            __syncthreads();
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                fmn = fmn < rmn[w] ? fmn : rmn[w];
                fmx = fmx > rmx[w] ? fmx : rmx[w];
            }
            if (fmn != fmx) {  // block-uniform; equal keys take the record path below
                const int fhi = 31 - __clz(fmn ^ fmx);
                const int flo = fhi > 10 ? fhi - 10 : 0;
                const uint32_t fdm = (2u << (fhi - flo)) - 1u;  // digit = bits flo..fhi
                for_keys(tid, total, kThreads, [&](int, uint32_t k) { atomicAdd(&h[(k >> flo) & fdm], 1u); });
                __syncthreads();
                find_bin_desc(h, kHistBins, (uint32_t)a.N, &sel_bin, &above, red);
                // the bucket's lower edge: the common bits above fhi, the digit, zeros below
                const uint32_t high = fhi == 31 ? 0u : (fmn & ~((2u << fhi) - 1u));
                const uint32_t edge = high | ((uint32_t)sel_bin << flo);
                const int per = (total + kThreads - 1) / kThreads;
                const int f0 = min(total, tid * per), f1 = min(total, f0 + per);
                int fc = 0;
                for_keys(f0, f1, 1, [&](int, uint32_t k) { fc += k >= edge; });
                int ftot;
                int fo = block_excl_scan<kWaves>(fc, red, &ftot);
                if (ftot <= kRefineCap) {  // block-uniform
                    for (int base = f0; base < f1; base += SU) {  // SU entries' loads together
                        int2 v[SU];
                        int sg[SU];
#pragma unroll
                        for (int u = 0; u < SU; ++u) {
                            const int i = min(f1 - 1, base + u);
                            sg[u] = seg_of(i);
                            v[u] = *entry_ptr(sg[u], i);
                        }
#pragma unroll
                        for (int u = 0; u < SU; ++u) {
                            const uint32_t k = fkey(__int_as_float(v[u].y));
                            if (base + u < f1 && k >= edge) {
                                epos[fo] = v[u].x;
                                ekey[fo] = k;
                                eseg[fo] = (uint16_t)sg[u];
                                ++fo;
                            }
                        }
                    }
                    total = ftot;
                    staged = true;
                }
            }
            __syncthreads();  // every read of rmn / rmx and h above is done
        }

        uint32_t fmn = 0xffffffffu, fmx = 0u;
        for_keys(tid, total, kThreads, [&](int, uint32_t k) {
            fmn = fmn < k ? fmn : k;
            fmx = fmx > k ? fmx : k;
        });
        fmn = ~wave_max_u32_dpp(~fmn);
        fmx = wave_max_u32_dpp(fmx);
        if (lane == 0) {
            rmn[wave] = fmn;
            rmx[wave] = fmx;
        }
        __syncthreads();
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            kmn = kmn < rmn[w] ? kmn : rmn[w];
            kmx = kmx > rmx[w] ? kmx : rmx[w];
        }
    }  // !fast

    // The listed keys agree above their highest differing bit hi.  Radix
    // digits of up to 11 bits go down from there (2048-bin LDS histograms)
    // until the bucket holding the wanted rank has at most kThreads keys,
    // which are then ranked against each other, or until every bit is fixed.
    if (tid == 0) sel_key = kmn;  // (the bound lists at least N keys; this is never kept)
    // keys that agree with p above bit h (h = -1: equal keys)
    auto agrees = [](uint32_t k, uint32_t p, int h) { return ((uint64_t)(k ^ p) >> (h + 1)) == 0; };
    uint32_t tkey = kmn;  // every listed key equal
    if (kmn != kmx) {     // block-uniform
        int hi = 31 - __clz(kmn ^ kmx);
        uint32_t pfx = kmn;            // right above bit hi; lower bits fixed digit by digit
        uint32_t rank = (uint32_t)a.N;  // rank wanted among the keys that agree with pfx above hi
        int cnt = total;
        while (hi >= 0 && cnt > kThreads) {  // block-uniform
            const int lo = hi > 10 ? hi - 10 : 0;
            const uint32_t dm = (2u << (hi - lo)) - 1u;  // digit = bits lo..hi
            __syncthreads();  // every read of the previous digit's histogram is done
            for (int i = tid; i < kHistBins; i += kThreads) h[i] = 0u;
            __syncthreads();
            for_keys(tid, total, kThreads, [&](int, uint32_t k) {
                if (agrees(k, pfx, hi)) atomicAdd(&h[(k >> lo) & dm], 1u);
            });
            __syncthreads();
            find_bin_desc(h, kHistBins, rank, &sel_bin, &above, red);
            const uint32_t bin = (uint32_t)sel_bin;
            rank -= above;
            cnt = (int)h[bin];
            pfx = (pfx & ~(dm << lo)) | (bin << lo);
            hi = lo - 1;
        }
        if (hi < 0) {
            tkey = pfx;  // every bit fixed: the bucket holds equal keys
        } else {
            // the cnt keys that agree with pfx above hi (any order), each
            // ranked against the others
            for_keys(tid, total, kThreads, [&](int, uint32_t k) {
                if (agrees(k, pfx, hi)) cand[atomicAdd(&ncand, 1)] = k;
            });
            __syncthreads();
            if (tid < cnt) {
                const uint32_t mine = cand[tid];
                int gt = 0, ge = 0;
                for (int q = 0; q < cnt; ++q) {
                    const uint32_t o = cand[q];
                    gt += o > mine;
                    ge += o >= mine;
                }
                if (gt < (int)rank && (int)rank <= ge) sel_key = mine;  // equal keys write equal values
            }
            __syncthreads();
            tkey = sel_key;
        }
    }
    if (tid == 0) a.tau[row] = fkey_inv(tkey);

    if (fast) {
        // the thread's segment: its survivors' rank in record order (one scan),
        // the first N of the row to pivot, and its record rewritten in place
        // from the staged copy
        int cnt = 0;
        for (int k = 0; k < f_n; ++k) cnt += ekey[f_off + k] >= tkey;
        int tot_pass;
        int r = block_excl_scan<kWaves>(cnt, red, &tot_pass);
        int32_t *P = a.pivot + (int64_t)row * a.N;
        int2 *dst = (int2 *)(rb + (int64_t)tid * a.seg_w) + 1;
        int kept = 0;
        for (int k = 0; k < f_n; ++k) {
            const uint32_t key = ekey[f_off + k];
            if (key >= tkey) {
                const int t = epos[f_off + k];
                if (r < a.N) P[r] = t;
                dst[kept++] = int2{t, __float_as_int(fkey_inv(key))};
                ++r;
            }
        }
        if (tid < a.n_sub) rb[(int64_t)tid * a.seg_w] = kept;  // new count; the key word stays
        return;
    }

    // survivors per segment, their record-order ranks, the first N -> pivot
    const int per = (total + kThreads - 1) / kThreads;
    const int i0 = min(total, tid * per), i1 = min(total, i0 + per);
    int cnt = 0;
    for_keys(i0, i1, 1, [&](int i, uint32_t k) {
        if (k >= tkey) {
            ++cnt;
            if (staged) atomicAdd(&pcnt[eseg[i]], 1);
        }
    });
    int tot_pass;
    const int r0 = block_excl_scan<kWaves>(cnt, red, &tot_pass);
    int r = r0;
    int32_t *P = a.pivot + (int64_t)row * a.N;
    if (staged) {
        for (int i = i0; i < i1 && r < a.N; ++i)
            if (ekey[i] >= tkey) P[r++] = epos[i];
    } else {
        for (int base = i0; base < i1 && r < a.N; base += SU) {  // SU entries' loads together
            int2 v[SU];
#pragma unroll
            for (int u = 0; u < SU; ++u) {
                const int i = min(i1 - 1, base + u);
                v[u] = *entry_ptr(seg_of(i), i);
            }
#pragma unroll
            for (int u = 0; u < SU; ++u)
                if (base + u < i1 && r < a.N && fkey(__int_as_float(v[u].y)) >= tkey) P[r++] = v[u].x;
        }
    }
    if (staged) {
        // survivors before each segment -> in-place rewrite from the LDS copy
        int pm = 0, pc[SPT];
#pragma unroll
        for (int i = 0; i < SPT; ++i) {
            const int sgi = tid * SPT + i;
            pc[i] = sgi < a.n_sub ? pcnt[sgi] : 0;
            pm += pc[i];
        }
        int ptot;
        int pb = block_excl_scan<kWaves>(pm, red, &ptot);
#pragma unroll
        for (int i = 0; i < SPT; ++i) {
            const int sgi = tid * SPT + i;
            if (sgi < a.n_sub) {
                pbase[sgi] = pb;
                rb[(int64_t)sgi * a.seg_w] = pc[i];  // new count; the key word stays
            }
            pb += pc[i];
        }
        __syncthreads();
        int rr = r0;
        for (int i = i0; i < i1; ++i) {
            const uint32_t k = ekey[i];
            if (k >= tkey) {
                const int sgi = eseg[i];
                int2 *dst = (int2 *)(rb + (int64_t)sgi * a.seg_w) + 1 + (rr - pbase[sgi]);
                *dst = int2{epos[i], __float_as_int(fkey_inv(k))};
                ++rr;
            }
        }
    } else {
        // in place, one segment per wave at a time, 64 entries per round: a
        // round reads its entries before writing survivors to lower indices
        __syncthreads();  // every read of the walk above is done
        for (int sgi = wave; sgi < a.n_sub; sgi += kWaves) {
            const int n = soff[sgi + 1] - soff[sgi];
            int2 *e = (int2 *)(rb + (int64_t)sgi * a.seg_w) + 1;
            int kept = 0;
            for (int k0 = 0; k0 < n; k0 += kWave) {
                const int k = k0 + lane;
                const int2 v = k < n ? e[k] : int2{0, 0};
                const bool ps = k < n && fkey(__int_as_float(v.y)) >= tkey;
                const uint64_t m = ballot(ps);
                __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
                if (ps) e[kept + mbcnt_lt(m)] = v;
                kept += __popcll(m);
            }
            if (lane == 0) rb[(int64_t)sgi * a.seg_w] = kept;
        }
    }
}

// ------------------------------------------------------------------ cache append

struct AppendArgs {
    uint16_t *K, *V;               // [B][h_k][ld_kv][D], [B][h_v][ld_kv][D]
    const uint16_t *k_new, *v_new; // [B][h_k][D], [B][h_v][D]
    int B, h_k, h_v, d;
    int64_t ld_kv, pos;
};

// Write the new token's key and value rows at cache position pos: one lane
// per 16 bytes.
__global__ __launch_bounds__(kThreads) void k_append(AppendArgs a) {
    const int per = a.d / 8;  // 16-byte pieces per row
    const int64_t nk = (int64_t)a.B * a.h_k * per, nv = (int64_t)a.B * a.h_v * per;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nk + nv;
         i += (int64_t)gridDim.x * kThreads) {
        const bool isk = i < nk;
        const int64_t x = isk ? i : i - nk;
        const int64_t head = x / per, c = x % per;  // head = b * h + g
        const uint16_t *src = (isk ? a.k_new : a.v_new) + head * a.d + c * 8;
        uint16_t *dst = (isk ? a.K : a.V) + (head * a.ld_kv + a.pos) * a.d + c * 8;
        *(u32x4 *)dst = ld16(src);
    }
}

// ------------------------------------------------------------------ read probe

// Plain streaming read (the reference rate for the streaming kernels): block
// i reads a contiguous range, each lane eight 16-byte loads per round that
// are kThreads * 16 bytes apart, and folds the words it read with XOR.
// Positions past the range are clamped to its last item and masked, so the
// loads carry no branches.
__global__ __launch_bounds__(kSelThreads) void k_read_probe(const u32x4 *p, int64_t n16, int64_t per,
                                                          uint32_t *sink) {
    __shared__ uint32_t red[kSelWaves];
    const int64_t beg = (int64_t)blockIdx.x * per;
    const int64_t end = min(n16, beg + per);
    uint32_t acc = 0u;
    for (int64_t i = beg + threadIdx.x; i < end; i += kSelThreads * 8) {
        u32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int64_t k = i + (int64_t)u * kSelThreads;
            v[u] = ld16_stream(p + (k < end ? k : end - 1));
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (i + (int64_t)u * kSelThreads < end) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    for (int o = 32; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = 0u;
#pragma unroll
        for (int w = 0; w < kSelWaves; ++w) r ^= red[w];
        sink[blockIdx.x] = r;
    }
}

// Plain streaming read with a chosen launch shape (the search for the best
// cold-read pattern): WAVES waves per workgroup, UNR 16-byte non-temporal
// loads in flight per lane.  CHUNKED: workgroup i reads the contiguous range
// [i*per, (i+1)*per) of 16-byte items, its lanes consecutive; else the
// workgroups take consecutive runs of WAVES*64*UNR items in turn (grid-
// strided).  Items past the end are clamped to the last item and masked.
// Each workgroup folds the words it read with XOR into
// sink[blockIdx.x % SAGA_PROBE_SINK_WORDS] (atomically).
template <int WAVES, int UNR, bool CHUNKED>
__global__ __launch_bounds__(WAVES * kWave) void k_read_probe_shape(const u32x4 *p, int64_t n16,
                                                                   int64_t per, uint32_t *sink,
                                                                   int sink_words) {
    constexpr int T = WAVES * kWave;
    uint32_t acc = 0u;
    const int64_t beg = CHUNKED ? (int64_t)blockIdx.x * per : (int64_t)blockIdx.x * T * UNR;
    const int64_t end = CHUNKED ? min(n16, beg + per) : n16;
    const int64_t stride = CHUNKED ? (int64_t)T * UNR : (int64_t)gridDim.x * T * UNR;
    for (int64_t i = beg + threadIdx.x; i < end; i += stride) {
        u32x4 v[UNR];
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            const int64_t k = i + (int64_t)u * T;
            v[u] = ld16_stream(p + (k < end ? k : end - 1));
        }
#pragma unroll
        for (int u = 0; u < UNR; ++u)
            if (i + (int64_t)u * T < end) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    for (int o = 32; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o);
    if ((threadIdx.x & 63) == 0) atomicXor(sink + blockIdx.x % sink_words, acc);
}

// ------------------------------------------------------------------ dense

struct DenseArgs {
    const uint16_t *Q, *K, *V;
    int B, h_q, h_k, h_v;  // K [B][h_k][l_kv][D], V [B][h_v][l_kv][D]
    int n_chunk;
    int n_vsub;            // value-head subsets (of NV heads) per key head
    int64_t l_kv, chunk_len;
    float scale_log2;      // log2(e) / sqrt(d)
    float *partial;        // [rows][n_chunk][D + 4]: m (log2 units), l, -, -, o[D]
};

// Dense split-KV decode with key head floor(j*h_k/h_q) and value head
// floor(j*h_v/h_q): one workgroup per (b, key head, value-head subset,
// chunk).  Scores by MFMA as in k_select; online softmax in base 2 per wave;
// P*V on the VALU (each lane owns 8 columns of a few rows of every tile, of
// each of the subset's NV value heads; a query head adds the rows of its own
// value head, a wave-uniform choice).  NV = 1 is dense GQA (h_k = h_v).
// RUN > 0: every value head serves RUN consecutive query heads and the
// block's first query head starts such a run (h_q/h_v = RUN and h_k divides
// h_v), so block head h uses subset value head h / RUN, known at compile
// time; RUN = 0 looks the value head up per head at run time, one branch per
// head and V row.
template <int D, int GMAX, int NV, int RUN>
__global__ __launch_bounds__(kThreads) void k_dense(DenseArgs a) {
    constexpr int KS = D / 32;
    constexpr int U = NV == 1 ? SAGA_DENSE_U * 64 / D : 1;
    constexpr int LPR = D / 8;          // lanes per V row
    constexpr int RPI = 64 / LPR;       // V rows per wave load
    constexpr int RPL = 16 / RPI;       // V rows per lane per tile
    constexpr bool kPingPong = GMAX <= 8;  // two tile buffers fit in registers
    __shared__ float p_lds[kWaves][U * 16][16];
    __shared__ float al_lds[kWaves][16];
    __shared__ float wm[kWaves][16], wl[kWaves][16];
    __shared__ float wo[kWaves][GMAX][D];

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int ln = lane & 15, lq = lane >> 4;
    const int chunk = blockIdx.x % a.n_chunk;
    const int vsub = (blockIdx.x / a.n_chunk) % a.n_vsub;
    const int bg = blockIdx.x / a.n_chunk / a.n_vsub;
    const int b = bg / a.h_k, g = bg % a.h_k;
    int j_lo = group_lo(g, a.h_q, a.h_k), j_hi = group_lo(g + 1, a.h_q, a.h_k);
    // this block's value heads [v_lo, v_lo + NV) and their query heads
    const int v_lo = j_lo * a.h_v / a.h_q + vsub * NV;  // j * h_v < 2^30 (h_q <= 32768)
    if (NV > 1 || a.n_vsub > 1) {
        j_lo = max(j_lo, group_lo(v_lo, a.h_q, a.h_v));
        j_hi = min(j_hi, group_lo(v_lo + NV, a.h_q, a.h_v));
    }
    const int G = j_hi - j_lo;
    if (G <= 0) return;  // whole block: a subset past the group's value heads
    const int64_t t_begin = (int64_t)chunk * a.chunk_len;
    const int64_t t_end = min(a.l_kv, t_begin + a.chunk_len);
    auto kcol = [](int lq, int s) { return s * 32 + lq * 8; };  // same d-axis map for Q and K

    bf16x8 qop[KS];
    {
        const int j = j_lo + ln;
        const bool jv = ln < G;
        const uint16_t *qp = a.Q + ((int64_t)b * a.h_q + (jv ? j : j_lo)) * D;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            u32x4 r = ld16(qp + kcol(lq, s));
            if (!jv) r = u32x4{0u, 0u, 0u, 0u};
            qop[s] = as_bf16x8(r);
        }
    }
    float m_run = -INFINITY, l_run = 0.f;  // for head ln
    float o[GMAX][8];
#pragma unroll
    for (int h = 0; h < GMAX; ++h)
#pragma unroll
        for (int i = 0; i < 8; ++i) o[h][i] = 0.f;

    const uint16_t *Kb = a.K + (int64_t)bg * a.l_kv * D;
    const uint16_t *Vb[NV];
    int vix[GMAX];  // value head of each query head, within the subset
#pragma unroll
    for (int vi = 0; vi < NV; ++vi)
        Vb[vi] = a.V + ((int64_t)b * a.h_v + min(v_lo + vi, a.h_v - 1)) * a.l_kv * D;
    if constexpr (NV > 1 && RUN == 0) {
#pragma unroll
        for (int h = 0; h < GMAX; ++h)
            vix[h] = (j_lo + h) * a.h_v / a.h_q - v_lo;
    }
    const int vr = lane / LPR, vc = (lane % LPR) * 8;
    const int64_t last = t_end - 1;

    // K and V tiles of one wave iteration; rows past the chunk are clamped to
    // its last row (their scores are set to -inf, so they weigh nothing).
    auto load_tiles = [&](u32x4 (&kr)[U][KS], u32x4 (&vv)[U][RPL][NV], int64_t t0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            int64_t row = t0 + u * 16 + ln;
            row = row < last ? row : last;
            const uint16_t *kp = Kb + row * D;
#pragma unroll
            for (int s = 0; s < KS; ++s) kr[u][s] = ld_k(kp + kcol(lq, s));
#pragma unroll
            for (int k = 0; k < RPL; ++k) {
                int64_t vrow = t0 + u * 16 + vr + k * RPI;
                vrow = vrow < last ? vrow : last;
#pragma unroll
                for (int vi = 0; vi < NV; ++vi) vv[u][k][vi] = ld_k(Vb[vi] + vrow * D + vc);
            }
        }
    };
    auto process = [&](const u32x4 (&kr)[U][KS], const u32x4 (&vv)[U][RPL][NV], int64_t t0) {
        float sc[U][4];
        float tmax = -INFINITY;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KS; ++s)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kr[u][s]), qop[s], acc, 0,
                                                              0, 0);
            const int64_t tr = t0 + u * 16 + lq * 4;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                sc[u][r] = (tr + r < t_end) ? acc[r] * a.scale_log2 : -INFINITY;
                tmax = fmaxf(tmax, sc[u][r]);
            }
        }
        tmax = fmaxf(tmax, __uint_as_float(from_xor16(__float_as_uint(tmax))));
        tmax = fmaxf(tmax, __uint_as_float(from_xor32(__float_as_uint(tmax))));
        const float m_new = fmaxf(m_run, tmax);
        const float alpha = exp2f(m_run - m_new);
        float psum = 0.f;
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float p = exp2f(sc[u][r] - m_new);
                psum += p;
                p_lds[wave][u * 16 + lq * 4 + r][ln] = p;
            }
        psum = add_xor<32>(add_xor<16>(psum));
        l_run = l_run * alpha + psum;
        m_run = m_new;
        if (lq == 0) al_lds[wave][ln] = alpha;
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int h = 0; h < GMAX; ++h) {
            const float al = al_lds[wave][h];
#pragma unroll
            for (int i = 0; i < 8; ++i) o[h][i] *= al;
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int k = 0; k < RPL; ++k)
#pragma unroll
                for (int vi = 0; vi < NV; ++vi) {
                    float vf[8];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        vf[2 * i] = bf_lo(vv[u][k][vi][i]);
                        vf[2 * i + 1] = bf_hi(vv[u][k][vi][i]);
                    }
                    const int rr = u * 16 + vr + k * RPI;
#pragma unroll
                    for (int h = 0; h < GMAX; ++h) {
                        if constexpr (NV > 1 && RUN > 0) {
                            if (h / RUN != vi) continue;  // resolved at compile time
                        } else if (NV > 1 && vix[h] != vi) {
                            continue;  // uniform: another value head
                        }
                        const float p = p_lds[wave][rr][h];
#pragma unroll
                        for (int i = 0; i < 8; ++i) o[h][i] += p * vf[i];
                    }
                }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
    };

    constexpr int64_t kStride = kWaves * 16 * U;
    int64_t t0 = t_begin + wave * 16 * U;
    if (t0 < t_end) {
        u32x4 ka[U][KS], va[U][RPL][NV];
        load_tiles(ka, va, t0);
        if constexpr (kPingPong) {
            u32x4 kb[U][KS], vb[U][RPL][NV];
            for (;;) {
                load_tiles(kb, vb, t0 + kStride);
                process(ka, va, t0);
                t0 += kStride;
                if (t0 >= t_end) break;
                load_tiles(ka, va, t0 + kStride);
                process(kb, vb, t0);
                t0 += kStride;
                if (t0 >= t_end) break;
            }
        } else {
            for (;;) {
                process(ka, va, t0);
                t0 += kStride;
                if (t0 >= t_end) break;
                load_tiles(ka, va, t0);
            }
        }
    }
    // combine the lanes of a wave that hold the same columns
#pragma unroll
    for (int h = 0; h < GMAX; ++h)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if constexpr (LPR <= 8) o[h][i] = add_xor<8>(o[h][i]);
            o[h][i] = add_xor<32>(add_xor<16>(o[h][i]));
        }
    if (lq == 0) {
        wm[wave][ln] = m_run;
        wl[wave][ln] = l_run;
    }
    if (lane < LPR)
#pragma unroll
        for (int h = 0; h < GMAX; ++h)
#pragma unroll
            for (int i = 0; i < 8; ++i) wo[wave][h][vc + i] = o[h][i];
    __syncthreads();
    // combine the waves, write this chunk's partial for each query head
    for (int x = threadIdx.x; x < G * D; x += kThreads) {
        const int h = x / D, c = x % D;
        float M = -INFINITY;
#pragma unroll
        for (int q = 0; q < kWaves; ++q) M = fmaxf(M, wm[q][h]);
        float L = 0.f, acc = 0.f;
#pragma unroll
        for (int q = 0; q < kWaves; ++q) {
            const float f = (wm[q][h] == -INFINITY) ? 0.f : exp2f(wm[q][h] - M);
            L += f * wl[q][h];
            acc += f * wo[q][h][c];
        }
        float *part = a.partial + (((int64_t)b * a.h_q + j_lo + h) * a.n_chunk + chunk) * (D + 4);
        part[4 + c] = acc;
        if (c == 0) {
            part[0] = M;
            part[1] = L;
        }
    }
}

struct DenseMergeArgs {
    const float *partial;
    int n_chunk;
    float *O;
};

template <int D>
__global__ __launch_bounds__(kThreads) void k_dense_merge(DenseMergeArgs a) {
    constexpr int NG = kThreads / D;
    __shared__ float sm[NG][D];
    __shared__ float sl[NG];
    __shared__ float smax[kWaves];
    const int row = blockIdx.x;
    const float *pr = a.partial + (int64_t)row * a.n_chunk * (D + 4);
    float M = -INFINITY;
    for (int k = threadIdx.x; k < a.n_chunk; k += kThreads) M = fmaxf(M, pr[(int64_t)k * (D + 4)]);
    M = wave_max(M);
    if ((threadIdx.x & 63) == 0) smax[threadIdx.x >> 6] = M;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kWaves; ++q) M = fmaxf(M, smax[q]);
    const int c = threadIdx.x % D, grp = threadIdx.x / D;
    float acc = 0.f, L = 0.f;
    // the group's chunks grp, grp + NG, ... in order, UNR at a time with all
    // their loads in flight
    constexpr int UNR = 8;
    for (int k0 = grp; k0 < a.n_chunk; k0 += NG * UNR) {
        float mk[UNR], vk[UNR], lk[UNR];
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            const int k = k0 + u * NG;
            const bool ok = k < a.n_chunk;
            const float *pk = pr + (int64_t)(ok ? k : k0) * (D + 4);
            mk[u] = ok ? pk[0] : -INFINITY;
            vk[u] = pk[4 + c];
            lk[u] = pk[1];
        }
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            const float f = (mk[u] == -INFINITY) ? 0.f : exp2f(mk[u] - M);
            acc += f * vk[u];
            L += f * lk[u];
        }
    }
    sm[grp][c] = acc;
    if (c == 0) sl[grp] = L;
    __syncthreads();
    if (threadIdx.x < D) {
        float s = 0.f, l = 0.f;
#pragma unroll
        for (int q = 0; q < NG; ++q) {
            s += sm[q][threadIdx.x];
            l += sl[q];
        }
        a.O[(int64_t)row * D + threadIdx.x] = l > 0.f ? s / l : 0.f;
    }
}

// ------------------------------------------------------------------ misc

__global__ void k_fill_u32(uint32_t *p, int64_t n, uint32_t v) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = v;
}

__global__ void k_fill_u8(uint8_t *p, int64_t n, uint8_t v) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = v;
}

struct MaskArgs {
    const int32_t *seg;
    int n_sub;
    int64_t sub_cap, seg_w, l_kv;
    uint8_t *mask;  // [rows][l_kv]
};

// One block per (row, segment): set mask[row][t] for every listed t.
__global__ __launch_bounds__(kThreads) void k_mask(MaskArgs a) {
    const int64_t rs = blockIdx.x;  // row * n_sub + sub
    const int64_t row = rs / a.n_sub;
    const int2 *rec = (const int2 *)(a.seg + rs * a.seg_w);
    int64_t cnt = rec[0].x;
    cnt = cnt < 0 ? 0 : (cnt > a.sub_cap ? a.sub_cap : cnt);  // never trust stale contents
    for (int64_t i = threadIdx.x; i < cnt; i += kThreads) {
        const int32_t t = rec[1 + i].x;
        if (t >= 0 && t < a.l_kv) a.mask[row * a.l_kv + t] = 1;
    }
}

}  // namespace saga
