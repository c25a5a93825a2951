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
//                        survivors through LDS into per-(row, sub-chunk)
//                        segments.                       [HBM-bound, hot]
//   k_attend             per row: max and count from the segment headers,
//                        softmax weights, gather of the survivors' V rows,
//                        fp32 accumulation, deterministic cross-block merge.
// Refresh (every R steps) instead runs:
//   k_select<.., true>   same score pass, writes fp32 A
//   k_hist / k_select1 / k_collect / k_select_final   exact radix select
//   k_compact            A >= tau into the same segments, then k_attend.
// Dense GQA baseline: k_dense (split-KV online softmax) + k_dense_merge.
#pragma once

#include "saga_device.hpp"

namespace saga {

constexpr int kWaves = 4;     // waves per workgroup of the streaming kernels
constexpr int kThreads = kWaves * kWave;
constexpr int kCapW = 32;     // LDS staging slots per (wave, query head)
constexpr int kMaxSub = 4096; // max segments per row
constexpr int kHistBins = 2048;

// ------------------------------------------------------------------ select

struct SelectArgs {
    const uint16_t *Q;   // bf16 [B][h_q][D]
    const uint16_t *K;   // bf16 [B][h_k][l_kv][D]
    const float *tau;    // [B*h_q]            (compare mode)
    float *A;            // [B*h_q][ld_a]      (materialize mode)
    int64_t ld_a;
    int B, h_q, h_k;
    int n_chunk;
    int64_t l_kv, chunk_len;
    float scale;
    int32_t *seg_t;      // [rows][n_sub][sub_cap]
    float *seg_s;
    int32_t *seg_count;  // [rows][n_sub]
    uint32_t *seg_maxkey;
    int n_sub;
    int64_t sub_cap;
};

// One workgroup = (batch b, key head g, chunk of cache positions).  Each wave
// takes 16-row tiles of K, U tiles at a time, interleaved across the 4 waves.
// MFMA 16x16x32 bf16: A operand = 16 K rows (M = position), B operand = the
// group's query heads (N = head, padded to 16 per N-tile), K dim = d.  Lane
// l loads d/2 contiguous bytes of row l%16 (bytes (l/16)*d/2 ...), and the
// query operand uses the same permutation of the d axis, so each lane issues
// 16-byte loads and the whole tile is a contiguous 16*d*2-byte block.
// Output: lane l holds rows 4*(l/16)+r, r = 0..3, of query head l%16.
template <int D, int NT, bool MATERIALIZE>
__global__ __launch_bounds__(kThreads) void k_select(SelectArgs a) {
    constexpr int KS = D / 32;             // MFMA k-steps per row
    constexpr int U = (D == 64) ? 4 : 2;   // tiles per wave iteration (128 B per lane)
    constexpr int QW = D / 4;              // elements of a row per lane quarter
    __shared__ int32_t st_t[MATERIALIZE ? 1 : kWaves][MATERIALIZE ? 1 : NT * 16][kCapW];
    __shared__ float st_s[MATERIALIZE ? 1 : kWaves][MATERIALIZE ? 1 : NT * 16][kCapW];

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int ln = lane & 15, lq = lane >> 4;
    const int chunk = blockIdx.x % a.n_chunk;
    const int bg = blockIdx.x / a.n_chunk;
    const int b = bg / a.h_k, g = bg % a.h_k;
    const int j_lo = group_lo(g, a.h_q, a.h_k), j_hi = group_lo(g + 1, a.h_q, a.h_k);
    const int64_t t_begin = (int64_t)chunk * a.chunk_len;
    const int64_t t_end = min(a.l_kv, t_begin + a.chunk_len);

    bf16x8 qop[NT][KS];
    float tau_l[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int j = j_lo + nt * 16 + ln;
        const bool jv = j < j_hi;
        const uint16_t *qp = a.Q + ((int64_t)b * a.h_q + (jv ? j : j_lo)) * D + lq * QW;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            u32x4 r = ld16(qp + s * 8);
            if (!jv) r = u32x4{0u, 0u, 0u, 0u};
            qop[nt][s] = as_bf16x8(r);
        }
        if (!MATERIALIZE) tau_l[nt] = jv ? a.tau[(int64_t)b * a.h_q + j] : INFINITY;
    }

    int staged[NT], flushed[NT];
    uint32_t mkey[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) staged[nt] = flushed[nt] = 0, mkey[nt] = 0u;

    const int sub = chunk * kWaves + wave;
    const uint64_t head_mask = 0x0001000100010001ull << ln;
    const uint64_t lt_mask = (1ull << lane) - 1ull;
    const uint16_t *Kb = a.K + (int64_t)bg * a.l_kv * D;

    auto flush = [&]() {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int j = j_lo + nt * 16 + ln;
            if (j < j_hi) {
                const int64_t base =
                    (((int64_t)b * a.h_q + j) * a.n_sub + sub) * a.sub_cap + flushed[nt];
                for (int i = lq; i < staged[nt]; i += 4) {
                    a.seg_t[base + i] = st_t[wave][nt * 16 + ln][i];
                    a.seg_s[base + i] = st_s[wave][nt * 16 + ln][i];
                }
            }
            flushed[nt] += staged[nt];
            staged[nt] = 0;
        }
    };

    for (int64_t t0 = t_begin + wave * 16 * U; t0 < t_end; t0 += kWaves * 16 * U) {
        u32x4 kr[U][KS];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t row = t0 + u * 16 + ln;
            const uint16_t *kp = Kb + row * D + lq * QW;
#pragma unroll
            for (int s = 0; s < KS; ++s)
                kr[u][s] = (row < t_end) ? ld16_stream(kp + s * 8) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t tr = t0 + u * 16 + lq * 4;  // position of acc[0]
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
                        if (tr + 3 < t_end) {
                            *(f32x4 *)Ap = f32x4{sc[0], sc[1], sc[2], sc[3]};
                        } else {
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                if (tr + r < t_end) Ap[r] = sc[r];
                        }
                    }
                } else {
                    bool pr[4];
                    uint64_t m[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        pr[r] = (tr + r < t_end) && (sc[r] >= tau_l[nt]);
                        m[r] = ballot(pr[r]);
                    }
                    if ((m[0] | m[1] | m[2] | m[3]) != 0ull) {
                        int before = 0;
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            if (pr[r]) {
                                const int rank = staged[nt] + before +
                                                 __popcll(m[r] & head_mask & lt_mask);
                                st_t[wave][nt * 16 + ln][rank] = (int32_t)(tr + r);
                                st_s[wave][nt * 16 + ln][rank] = sc[r];
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
    }
    if (!MATERIALIZE) {
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        flush();
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            uint32_t mk = mkey[nt];
            uint32_t o = __shfl_xor(mk, 16);
            mk = mk > o ? mk : o;
            o = __shfl_xor(mk, 32);
            mk = mk > o ? mk : o;
            const int j = j_lo + nt * 16 + ln;
            if (lq == 0 && j < j_hi) {
                const int64_t h = ((int64_t)b * a.h_q + j) * a.n_sub + sub;
                a.seg_count[h] = flushed[nt];
                a.seg_maxkey[h] = mk;
            }
        }
    }
}

// ------------------------------------------------------------------ attend

struct AttendArgs {
    const int32_t *seg_t;
    const float *seg_s;
    const int32_t *seg_count;
    const uint32_t *seg_maxkey;
    int n_sub;
    int64_t sub_cap;
    const uint16_t *V;  // bf16 [B][h_v][l_kv][D]
    int B, h_q, h_v;
    int64_t l_kv;
    int pw;             // workgroups per row
    float *partial;     // [rows][pw][D + 4]
    uint32_t *ticket;   // [rows]
    float *O;           // [rows][D]
    int32_t *counts;    // [rows] or null
};

// Block-wide exclusive scan of v over kThreads threads; returns the prefix,
// *total receives the sum.  Uses red[kWaves] of LDS.
__device__ __forceinline__ int block_excl_scan(int v, int *red, int *total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    if (lane == 63) red[wave] = x;
    __syncthreads();
    int before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        before += (w < wave) ? red[w] : 0;
        tot += red[w];
    }
    __syncthreads();
    *total = tot;
    return before + x - v;
}

// One workgroup = (row, slice w of that row's survivors).  Every slice uses
// the row's exact maximum over the survivors (from the segment headers), so
// slice partials (sum of weights, weighted V sum) add directly; the last
// slice to finish adds them in slice order and normalises.
template <int D>
__global__ __launch_bounds__(kThreads) void k_attend(AttendArgs a) {
    constexpr int LPE = D / 8;        // lanes per survivor (16 B each)
    constexpr int EPB = kThreads / LPE;  // survivors per block round
    constexpr int UN = 4;
    __shared__ int pre[kMaxSub + 1];
    __shared__ int ired[kWaves];
    __shared__ uint32_t kred[kWaves];
    __shared__ float ored[kWaves][D];
    __shared__ float lred[kWaves];
    __shared__ int is_last;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int row = blockIdx.x / a.pw, w = blockIdx.x % a.pw;
    const int b = row / a.h_q, j = row % a.h_q;
    const int vh = (int)(((int64_t)j * a.h_v) / a.h_q);

    // segment headers -> exclusive prefix (pre[]), total count, max key
    const int per = (a.n_sub + kThreads - 1) / kThreads;
    const int s0 = min(a.n_sub, tid * per), s1 = min(a.n_sub, s0 + per);
    int csum = 0;
    uint32_t mk = 0u;
    const int64_t hbase = (int64_t)row * a.n_sub;
    for (int s = s0; s < s1; ++s) {
        csum += a.seg_count[hbase + s];
        const uint32_t k = a.seg_maxkey[hbase + s];
        mk = mk > k ? mk : k;
    }
    int total;
    int run = block_excl_scan(csum, ired, &total);
    for (int s = s0; s < s1; ++s) {
        pre[s] = run;
        run += a.seg_count[hbase + s];
    }
    if (tid == 0) pre[a.n_sub] = total;
    mk = wave_max_u32(mk);
    if (lane == 0) kred[wave] = mk;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kWaves; ++q) mk = mk > kred[q] ? mk : kred[q];
    const float M = fkey_inv(mk);
    const int64_t n = total;
    const int64_t lo = n * w / a.pw, hi = n * (w + 1) / a.pw;

    const int e_in = tid / LPE, cl = tid % LPE;
    const uint16_t *Vb = a.V + ((int64_t)b * a.h_v + vh) * a.l_kv * D + cl * 8;
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    float lsum = 0.f;
    for (int64_t e0 = lo; e0 < hi; e0 += (int64_t)EPB * UN) {
        int tt[UN];
        float pp[UN];
#pragma unroll
        for (int u = 0; u < UN; ++u) {
            const int64_t e = e0 + u * EPB + e_in;
            tt[u] = -1;
            pp[u] = 0.f;
            if (e < hi) {
                int lo_s = 0, hi_s = a.n_sub;  // largest s with pre[s] <= e
                while (hi_s - lo_s > 1) {
                    const int mid = (lo_s + hi_s) >> 1;
                    if (pre[mid] <= e) lo_s = mid; else hi_s = mid;
                }
                const int64_t idx = (hbase + lo_s) * a.sub_cap + (e - pre[lo_s]);
                tt[u] = a.seg_t[idx];
                pp[u] = expf(a.seg_s[idx] - M);
            }
        }
        u32x4 vv[UN];
#pragma unroll
        for (int u = 0; u < UN; ++u)
            vv[u] = tt[u] >= 0 ? ld16(Vb + (int64_t)tt[u] * D) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int u = 0; u < UN; ++u) {
            const float p = pp[u];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[2 * i] += p * bf_lo(vv[u][i]);
                acc[2 * i + 1] += p * bf_hi(vv[u][i]);
            }
            lsum += (cl == 0) ? p : 0.f;
        }
    }
    // reduce over the survivors handled by the lanes of a wave sharing cl
#pragma unroll
    for (int o = LPE; o < 64; o <<= 1)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += __shfl_xor(acc[i], o);
    lsum = wave_sum(lsum);
    if (lane < LPE)
#pragma unroll
        for (int i = 0; i < 8; ++i) ored[wave][lane * 8 + i] = acc[i];
    if (lane == 0) lred[wave] = lsum;
    __syncthreads();
    float *part = a.partial + ((int64_t)row * a.pw + w) * (D + 4);
    if (tid < D) {
        float s = 0.f;
#pragma unroll
        for (int q = 0; q < kWaves; ++q) s += ored[q][tid];
        __hip_atomic_store(part + 4 + tid, s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (tid == 0) {
        float s = 0.f;
#pragma unroll
        for (int q = 0; q < kWaves; ++q) s += lred[q];
        __hip_atomic_store(part, s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        const uint32_t old = atomicAdd(a.ticket + row, 1u);
        is_last = (old == (uint32_t)(a.pw - 1));
    }
    __syncthreads();
    if (!is_last) return;
    __threadfence();
    if (tid < D) {
        float so = 0.f, sl = 0.f;
        for (int q = 0; q < a.pw; ++q) {
            const float *pq = a.partial + ((int64_t)row * a.pw + q) * (D + 4);
            so += __hip_atomic_load(pq + 4 + tid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            sl += __hip_atomic_load(pq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        a.O[(int64_t)row * D + tid] = sl > 0.f ? so / sl : 0.f;
    }
    if (tid == 0) {
        if (a.counts) a.counts[row] = (int32_t)n;
        atomicExch(a.ticket + row, 0u);
    }
}

// ------------------------------------------------------------------ refresh

struct RadixArgs {
    const float *A;
    int64_t ld_a, l_kv, N;
    int rows;
    int bpr;          // blocks per row for the histogram/collect passes
    int64_t blk_len;  // positions per block
    uint32_t *hist;   // [rows][2048] (zero on entry, zero on exit)
    uint32_t *state;  // [rows][4]: prefix, rank within bucket, bucket size, fill counter
    uint32_t *cand;   // [rows][l_kv]
    float *tau;       // [rows]
};

// Digit 1: bits 31..21 of the order key, per-block LDS histogram.
__global__ __launch_bounds__(kThreads) void k_hist(RadixArgs a) {
    __shared__ uint32_t h[kHistBins];
    const int row = blockIdx.x / a.bpr, blk = blockIdx.x % a.bpr;
    for (int i = threadIdx.x; i < kHistBins; i += kThreads) h[i] = 0u;
    __syncthreads();
    const int64_t t0 = (int64_t)blk * a.blk_len, t1 = min(a.l_kv, t0 + a.blk_len);
    const float *Ar = a.A + (int64_t)row * a.ld_a;
    for (int64_t t = t0 + threadIdx.x; t < t1; t += kThreads) atomicAdd(&h[fkey(Ar[t]) >> 21], 1u);
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
    const uint32_t before = (uint32_t)block_excl_scan((int)c, red, &total);
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
    for (int i = threadIdx.x; i < kHistBins; i += kThreads) {
        h[i] = hg[i];
        hg[i] = 0u;  // leave the histogram cleared for the next refresh
    }
    __syncthreads();
    find_bin_desc(h, kHistBins, (uint32_t)a.N, &sel_bin, &above, red);
    if (threadIdx.x == 0) {
        uint32_t *st = a.state + (int64_t)row * 4;
        st[0] = (uint32_t)sel_bin;
        st[1] = (uint32_t)a.N - above;
        st[2] = h[sel_bin];
    }
}

// Gather the order keys of the bucket holding tau into cand[row].
__global__ __launch_bounds__(kThreads) void k_collect(RadixArgs a) {
    const int row = blockIdx.x / a.bpr, blk = blockIdx.x % a.bpr;
    const uint32_t prefix = a.state[(int64_t)row * 4 + 0];
    uint32_t *fill = a.state + (int64_t)row * 4 + 3;
    const int64_t t0 = (int64_t)blk * a.blk_len, t1 = min(a.l_kv, t0 + a.blk_len);
    const float *Ar = a.A + (int64_t)row * a.ld_a;
    uint32_t *cr = a.cand + (int64_t)row * a.l_kv;
    for (int64_t tb = t0; tb < t1; tb += kThreads) {
        const int64_t t = tb + threadIdx.x;
        uint32_t key = 0u;
        bool p = false;
        if (t < t1) {
            key = fkey(Ar[t]);
            p = (key >> 21) == prefix;
        }
        const uint64_t m = ballot(p);
        if (m) {
            uint32_t base = 0u;
            if ((threadIdx.x & 63) == 0) base = atomicAdd(fill, (uint32_t)__popcll(m));
            base = __shfl(base, 0);
            if (p) cr[base + mbcnt_lt(m)] = key;
        }
    }
}

// Finish the select on the bucket's keys: digits 20..10 then 9..0.
__global__ __launch_bounds__(kThreads) void k_select_final(RadixArgs a) {
    __shared__ uint32_t h[kHistBins];
    __shared__ int red[kWaves];
    __shared__ int sel_bin;
    __shared__ uint32_t above;
    const int row = blockIdx.x;
    uint32_t *st = a.state + (int64_t)row * 4;
    const uint32_t prefix = st[0], k = st[1], n = st[2];
    const uint32_t *cr = a.cand + (int64_t)row * a.l_kv;

    for (int i = threadIdx.x; i < kHistBins; i += kThreads) h[i] = 0u;
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
        st[3] = 0u;  // fill counter back to zero
    }
}

// Refresh step selection from the materialised scores: A >= tau into the
// same (row, sub-chunk) segments k_select writes.  Wave w of the block for
// (row, chunk) covers positions [chunk*chunk_len + w*sub_cap, ... + sub_cap).
struct CompactArgs {
    const float *A;
    int64_t ld_a, l_kv, chunk_len;
    int n_chunk;
    const float *tau;
    int32_t *seg_t;
    float *seg_s;
    int32_t *seg_count;
    uint32_t *seg_maxkey;
    int n_sub;
    int64_t sub_cap;
};

__global__ __launch_bounds__(kThreads) void k_compact(CompactArgs a) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int row = blockIdx.x / a.n_chunk, chunk = blockIdx.x % a.n_chunk;
    const int sub = chunk * kWaves + wave;
    const int64_t t0 = (int64_t)chunk * a.chunk_len + (int64_t)wave * a.sub_cap;
    const int64_t t1 = min(a.l_kv, t0 + a.sub_cap);
    const float tau = a.tau[row];
    const float *Ar = a.A + (int64_t)row * a.ld_a;
    const int64_t sbase = ((int64_t)row * a.n_sub + sub) * a.sub_cap;
    int cnt = 0;
    uint32_t mk = 0u;
    for (int64_t tb = t0; tb < t1; tb += 64) {
        const int64_t t = tb + lane;
        float s = 0.f;
        bool p = false;
        if (t < t1) {
            s = Ar[t];
            p = s >= tau;
        }
        const uint64_t m = ballot(p);
        if (p) {
            const int pos = cnt + mbcnt_lt(m);
            a.seg_t[sbase + pos] = (int32_t)t;
            a.seg_s[sbase + pos] = s;
            const uint32_t k = fkey(s);
            mk = mk > k ? mk : k;
        }
        cnt += __popcll(m);
    }
    mk = wave_max_u32(mk);
    if (lane == 0) {
        a.seg_count[(int64_t)row * a.n_sub + sub] = cnt;
        a.seg_maxkey[(int64_t)row * a.n_sub + sub] = mk;
    }
}

// ------------------------------------------------------------------ dense

struct DenseArgs {
    const uint16_t *Q, *K, *V;
    int B, h_q, h_kv;
    int n_chunk;
    int64_t l_kv, chunk_len;
    float scale_log2;  // log2(e) / sqrt(d)
    float *partial;    // [rows][n_chunk][D + 4]: m (log2 units), l, -, -, o[D]
};

// Dense GQA split-KV decode: one workgroup per (b, kv head, chunk).  Scores
// by MFMA as in k_select; online softmax in base 2 per wave; P*V on the VALU
// (each lane owns 8 columns of a few rows of every tile).
template <int D, int GMAX>
__global__ __launch_bounds__(kThreads) void k_dense(DenseArgs a) {
    constexpr int KS = D / 32;
    constexpr int U = (D == 64) ? 4 : 2;
    constexpr int QW = D / 4;
    constexpr int LPR = D / 8;          // lanes per V row
    constexpr int RPI = 64 / LPR;       // V rows per wave load
    constexpr int RPL = 16 / RPI;       // V rows per lane per tile
    __shared__ float p_lds[kWaves][U * 16][16];
    __shared__ float al_lds[kWaves][16];
    __shared__ float wm[kWaves][16], wl[kWaves][16];
    __shared__ float wo[kWaves][GMAX][D];

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int ln = lane & 15, lq = lane >> 4;
    const int chunk = blockIdx.x % a.n_chunk;
    const int bg = blockIdx.x / a.n_chunk;
    const int b = bg / a.h_kv, g = bg % a.h_kv;
    const int j_lo = group_lo(g, a.h_q, a.h_kv), j_hi = group_lo(g + 1, a.h_q, a.h_kv);
    const int G = j_hi - j_lo;
    const int64_t t_begin = (int64_t)chunk * a.chunk_len;
    const int64_t t_end = min(a.l_kv, t_begin + a.chunk_len);

    bf16x8 qop[KS];
    {
        const int j = j_lo + ln;
        const bool jv = ln < G;
        const uint16_t *qp = a.Q + ((int64_t)b * a.h_q + (jv ? j : j_lo)) * D + lq * QW;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            u32x4 r = ld16(qp + s * 8);
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
    const uint16_t *Vb = a.V + (int64_t)bg * a.l_kv * D;
    const int vr = lane / LPR, vc = (lane % LPR) * 8;

    for (int64_t t0 = t_begin + wave * 16 * U; t0 < t_end; t0 += kWaves * 16 * U) {
        u32x4 kr[U][KS];
        u32x4 vv[U][RPL];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t row = t0 + u * 16 + ln;
            const uint16_t *kp = Kb + row * D + lq * QW;
#pragma unroll
            for (int s = 0; s < KS; ++s)
                kr[u][s] = (row < t_end) ? ld16_stream(kp + s * 8) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int k = 0; k < RPL; ++k) {
                const int64_t vrow = t0 + u * 16 + vr + k * RPI;
                vv[u][k] = (vrow < t_end) ? ld16_stream(Vb + vrow * D + vc)
                                          : u32x4{0u, 0u, 0u, 0u};
            }
        }
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
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
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
        psum += __shfl_xor(psum, 16);
        psum += __shfl_xor(psum, 32);
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
            for (int k = 0; k < RPL; ++k) {
                float vf[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    vf[2 * i] = bf_lo(vv[u][k][i]);
                    vf[2 * i + 1] = bf_hi(vv[u][k][i]);
                }
                const int rr = u * 16 + vr + k * RPI;
#pragma unroll
                for (int h = 0; h < GMAX; ++h) {
                    const float p = p_lds[wave][rr][h];
#pragma unroll
                    for (int i = 0; i < 8; ++i) o[h][i] += p * vf[i];
                }
            }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
    }
    // combine the lanes of a wave that hold the same columns
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1)
#pragma unroll
        for (int h = 0; h < GMAX; ++h)
#pragma unroll
            for (int i = 0; i < 8; ++i) o[h][i] += __shfl_xor(o[h][i], off);
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
    for (int k = grp; k < a.n_chunk; k += NG) {
        const float *pk = pr + (int64_t)k * (D + 4);
        const float mk = pk[0];
        const float f = (mk == -INFINITY) ? 0.f : exp2f(mk - M);
        acc += f * pk[4 + c];
        L += f * pk[1];
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
    const int32_t *seg_t;
    const int32_t *seg_count;
    int n_sub;
    int64_t sub_cap, l_kv;
    uint8_t *mask;  // [rows][l_kv]
};

// One block per (row, segment): set mask[row][t] for every listed t.
__global__ __launch_bounds__(kThreads) void k_mask(MaskArgs a) {
    const int64_t rs = blockIdx.x;  // row * n_sub + sub
    const int64_t row = rs / a.n_sub;
    int64_t cnt = a.seg_count[rs];
    cnt = cnt < 0 ? 0 : (cnt > a.sub_cap ? a.sub_cap : cnt);  // never trust stale contents
    const int32_t *st = a.seg_t + rs * a.sub_cap;
    for (int64_t i = threadIdx.x; i < cnt; i += kThreads) {
        const int32_t t = st[i];
        if (t >= 0 && t < a.l_kv) a.mask[row * a.l_kv + t] = 1;
    }
}

}  // namespace saga
