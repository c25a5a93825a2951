// saga.hip -- C-ABI host library for SAGA + Atop-N decode attention on
// MI355X (gfx950).  Validates arguments, lays out the caller's workspace,
// and enqueues the kernels of saga_kernels.hpp on the caller's stream.
// Declarations and the contract of every entry point: include/saga.h.
#include <atomic>
#include <mutex>
#include <hip/hip_runtime.h>

#include <math.h>

#include <algorithm>
#include <stdint.h>
#include <string.h>

#include "../../include/saga.h"
#include "saga_kernels.hpp"

namespace {

using namespace saga;

#ifndef SAGA_SELECT_BLOCKS
#define SAGA_SELECT_BLOCKS 256
#endif
constexpr int kTargetSelectBlocks = SAGA_SELECT_BLOCKS;  // streaming blocks per launch
// Head-index products (g * h_q, j * h_v) stay below 2^30 in the kernels' 32-bit
// arithmetic.
constexpr int kMaxQueryHeads = 32768;
#ifndef SAGA_ATTEND_ROW
#define SAGA_ATTEND_ROW 1  // k_attend_row where the column-split grid is two blocks per CU or more
#endif
#ifndef SAGA_DENSE_BLOCKS
#define SAGA_DENSE_BLOCKS 512
#endif
constexpr int kTargetDenseBlocks = SAGA_DENSE_BLOCKS;  // dense baseline blocks per launch
constexpr int64_t kChunkUnit = kSelWaves * 16 * SAGA_SELECT_U;  // chunk_len granularity: one wave-iteration stride of the select block
constexpr int64_t kDenseChunkUnit = 256;  // dense chunk granularity: whole wave iterations of k_dense
static_assert(kDenseChunkUnit % (kWaves * 16 * SAGA_DENSE_U) == 0, "dense chunk unit");
constexpr int64_t kHistBlock = kHistBlockMax;  // positions per histogram/collect block
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct Plan {
    int B, h_q, h_k, h_v, d;
    int64_t l_kv, N;
    int rows, gmax, nt;
    int u;  // k_select tiles per wave iteration (a record group is 16 u rows)
    int64_t chunk_len;
    int n_chunk, n_sub;
    int64_t sub_cap;
    int64_t ld_a;
    int64_t ld_kv;  // rows per head in the K and V caches (>= l_kv)
    int hist_bpr;
    // byte offsets into the workspace
    size_t off_hist, off_state, off_pi, counters_end;
    int64_t grp;  // rows per k_select wave iteration (16 * U): the record order's groups
    int64_t seg_w;
    size_t off_seg, off_scores, off_cand;
    size_t total;
};

int check_shape(int B, int h_q, int h_k, int h_v, int d, int64_t l_kv, int64_t N) {
    if (B < 1 || h_q < 1 || h_k < 1 || h_v < 1 || l_kv < 1 || N < 1) return SAGA_ERR_INVALID_ARG;
    if (h_k > h_v || h_v > h_q) return SAGA_ERR_INVALID_ARG;
    if (N > l_kv) return SAGA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return SAGA_ERR_UNSUPPORTED;
    if (ceil_div(h_q, h_k) > 64) return SAGA_ERR_UNSUPPORTED;
    if (l_kv * (int64_t)d * 2 >= (int64_t(1) << 31)) return SAGA_ERR_UNSUPPORTED;
    if ((int64_t)B * h_q >= (int64_t(1) << 20)) return SAGA_ERR_UNSUPPORTED;
    if (h_q > kMaxQueryHeads) return SAGA_ERR_UNSUPPORTED;
    return SAGA_OK;
}

// Chunk granularity of the short-cache plan: one 16-row tile for each of the
// lower four waves (the upper four then have no rows and are not launched).
constexpr int64_t kShortUnit = kWaves * 16;

// Short cache: chunks of one streaming unit (kChunkUnit rows) would leave
// compute units idle, so the plan takes 64-row chunk units instead -- up to
// kTargetSelectBlocks blocks.  Monotone in l_kv: the short plan's chunks are
// never longer than kChunkUnit rows, the streaming plan's never shorter.
bool short_plan(int64_t pairs, int64_t l_kv) {
    return ceil_div(pairs * l_kv, kTargetSelectBlocks) <= kChunkUnit;
}

// k_select tiles per wave iteration: one on the short plan, else the
// streaming choice (SAGA_SELECT_U, one by default).  Chunk lengths are
// multiples of kWaves record groups either way (the record order needs it).
int select_u(int64_t pairs, int64_t l_kv, int d) {
    if (short_plan(pairs, l_kv)) return 1;
    return d == 64 ? select_tiles<64>() : select_tiles<128>();
}
static_assert(kShortUnit % (kWaves * 16) == 0, "short chunks: whole record groups per segment");
static_assert(kChunkUnit % (kWaves * 16 * select_tiles<64>()) == 0 &&
                  kChunkUnit % (kWaves * 16 * select_tiles<128>()) == 0,
              "streaming chunks: whole record groups per segment");

// Streaming split: about kTargetSelectBlocks blocks over all (b, key head)
// pairs, and at most kMaxSub/kWaves chunks per row (non-decreasing in l_kv).
int64_t chunk_len_for(int64_t pairs, int64_t l_kv) {
    const int64_t unit = short_plan(pairs, l_kv) ? kShortUnit : kChunkUnit;
    int64_t cl = ceil_div(ceil_div(pairs * l_kv, kTargetSelectBlocks), unit) * unit;
    const int64_t cl_min = ceil_div(ceil_div(l_kv, kMaxSub / kWaves), unit) * unit;
    if (cl < cl_min) cl = cl_min;
    if (cl < unit) cl = unit;
    return cl;
}

// cap > 0: a cache with room for cap rows per head, of which l_kv are in use;
// the workspace regions are then sized for any length up to cap (records:
// n_chunk * chunk_len < l_kv + chunk_len <= cap + chunk_len(cap)), so one
// workspace serves the whole growth.
int make_plan(int B, int h_q, int h_k, int h_v, int d, int64_t l_kv, int64_t N, Plan *p,
              int64_t cap = 0) {
    int st = check_shape(B, h_q, h_k, h_v, d, cap > 0 ? cap : l_kv, N);
    if (st != SAGA_OK) return st;
    if (cap > 0 && (l_kv < 1 || l_kv > cap || N > l_kv)) return SAGA_ERR_INVALID_ARG;
    memset(p, 0, sizeof *p);
    p->B = B, p->h_q = h_q, p->h_k = h_k, p->h_v = h_v, p->d = d, p->l_kv = l_kv, p->N = N;
    p->ld_kv = cap > 0 ? cap : l_kv;
    p->rows = B * h_q;
    p->gmax = (int)ceil_div(h_q, h_k);
    p->nt = p->gmax <= 16 ? 1 : (p->gmax <= 32 ? 2 : 4);
    const int64_t pairs = (int64_t)B * h_k;
    const int64_t cl = chunk_len_for(pairs, l_kv);
    p->chunk_len = cl;
    p->n_chunk = (int)ceil_div(l_kv, cl);
    p->n_sub = p->n_chunk * kWaves;
    p->sub_cap = cl / kWaves;
    p->u = select_u(pairs, l_kv, d);
    p->grp = 16 * p->u;
    p->ld_a = ceil_div(l_kv, 64) * 64;
    p->hist_bpr = (int)ceil_div(l_kv, kHistBlock);

    const size_t rows = (size_t)p->rows;
    size_t o = 0;
    p->off_hist = o;
    o = align_up(o + rows * kHistBins * sizeof(uint32_t));
    p->off_state = o;
    o = align_up(o + rows * 4 * sizeof(uint32_t));
    p->off_pi = o;   // fp32 [rows]: lower bounds of a refresh from a pivot
    o = align_up(o + rows * sizeof(float));
    p->counters_end = o;
    p->seg_w = seg_words(p->sub_cap);
    p->off_seg = o;
    size_t seg_bytes = rows * (size_t)p->n_sub * (size_t)p->seg_w * sizeof(int32_t);
    int64_t ld_a_max = p->ld_a, cand_len = l_kv;
    if (cap > 0) {
        const int64_t ccap = chunk_len_for(pairs, cap);
        seg_bytes = rows * (size_t)(2 * (cap + ccap) + 17 * (int64_t)kMaxSub) * sizeof(int32_t);
        ld_a_max = ceil_div(cap, 64) * 64;
        cand_len = cap;
    }
    o = align_up(o + seg_bytes);
    p->off_scores = o;
    o = align_up(o + rows * (size_t)ld_a_max * sizeof(float));
    p->off_cand = o;
    o = align_up(o + rows * (size_t)cand_len * sizeof(uint32_t));
    p->total = o;
    return SAGA_OK;
}

struct DensePlan {
    int rows, gmax, nv, n_vsub;
    int run;  // query heads per value head when every block's heads come in whole runs, else 0
    int64_t chunk_len;
    int n_chunk;
    size_t total;
};

int64_t host_group_lo(int64_t g, int64_t h_q, int64_t h_k) { return (g * h_q + h_k - 1) / h_k; }

// Dense decode plan for key heads h_k and value heads h_v (h_k = h_v: GQA).
// A block serves one key head's chunk and the query heads of up to nv of
// its group's value heads; groups with more value heads (or with more than
// 8 query heads over nv value heads) are split into n_vsub subsets, each
// reading the key rows again.
int make_dense_plan(int B, int h_q, int h_k, int h_v, int d, int64_t l_kv, DensePlan *p) {
    if (B < 1 || h_q < 1 || h_k < 1 || h_v < 1 || l_kv < 1) return SAGA_ERR_INVALID_ARG;
    if (h_k > h_v || h_v > h_q) return SAGA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return SAGA_ERR_UNSUPPORTED;
    if (l_kv * (int64_t)d * 2 >= (int64_t(1) << 31)) return SAGA_ERR_UNSUPPORTED;
    if ((int64_t)B * h_q >= (int64_t(1) << 20)) return SAGA_ERR_UNSUPPORTED;
    if (h_q > kMaxQueryHeads) return SAGA_ERR_UNSUPPORTED;
    auto vh = [&](int64_t j) { return j * h_v / h_q; };
    int64_t maxv = 1;
    for (int g = 0; g < h_k; ++g) {
        const int64_t jl = host_group_lo(g, h_q, h_k), jh = host_group_lo(g + 1, h_q, h_k);
        if (jh > jl) maxv = std::max(maxv, vh(jh - 1) - vh(jl) + 1);
    }
    // query heads per block for subsets of nv value heads
    auto block_heads = [&](int nv, int n_vsub) {
        int64_t gm = 0;
        for (int g = 0; g < h_k; ++g) {
            const int64_t jl = host_group_lo(g, h_q, h_k), jh = host_group_lo(g + 1, h_q, h_k);
            for (int vs = 0; vs < n_vsub; ++vs) {
                int64_t a = jl, bq = jh;
                if (nv > 1 || n_vsub > 1) {
                    const int64_t v_lo = vh(jl) + vs * nv;
                    a = std::max(jl, host_group_lo(v_lo, h_q, h_v));
                    bq = std::min(jh, host_group_lo(v_lo + nv, h_q, h_v));
                }
                gm = std::max(gm, bq - a);
            }
        }
        return gm;
    };
    // the largest subset (fewest key re-reads) whose blocks keep at most 8
    // query heads, the size that leaves registers for two tile buffers;
    // else the subset with the fewest query heads per block
    const int first = maxv == 1 ? 1 : (maxv == 2 ? 2 : 4);
    int64_t gmax = -1;
    for (int nv = first; nv >= 1; nv /= 2) {
        const int nvs = (int)ceil_div(maxv, nv);
        const int64_t gm = block_heads(nv, nvs);
        if (gmax < 0 || gm < gmax) {
            gmax = gm;
            p->nv = nv;
            p->n_vsub = nvs;
        }
        if (gm <= 8) break;
    }
    if (gmax > 16) return SAGA_ERR_UNSUPPORTED;
    p->rows = B * h_q;
    p->gmax = (int)gmax;
    // h_v | h_q and h_k | h_v: a group's first query head, and the first query
    // head of each subset, start a run of h_q/h_v heads on one value head
    p->run = (p->nv > 1 && h_q % h_v == 0 && h_v % h_k == 0) ? h_q / h_v : 0;
    const int64_t pairs = (int64_t)B * h_k * p->n_vsub;
    int64_t cl = ceil_div(ceil_div(pairs * l_kv, kTargetDenseBlocks), kDenseChunkUnit) * kDenseChunkUnit;
    const int64_t cl_min = ceil_div(ceil_div(l_kv, 4096), kDenseChunkUnit) * kDenseChunkUnit;
    if (cl < cl_min) cl = cl_min;
    if (cl < kDenseChunkUnit) cl = kDenseChunkUnit;
    p->chunk_len = cl;
    p->n_chunk = (int)ceil_div(l_kv, cl);
    p->total = align_up((size_t)p->rows * p->n_chunk * (d + 4) * sizeof(float));
    return SAGA_OK;
}

bool aligned(const void *ptr, size_t a) { return ((uintptr_t)ptr % a) == 0; }

int launch_status() { return hipGetLastError() == hipSuccess ? SAGA_OK : SAGA_ERR_HIP; }

// Compute units of the current device (cached per device; 256 on MI355X).
// Callers on several host threads may fill the cache at once; they store
// the same value.
int device_cus() {
    static std::atomic<int> cus[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int c = cus[dev].load(std::memory_order_relaxed);
    if (c == 0) {
        int n = 0;
        c = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0
                ? n : 256;
        cus[dev].store(c, std::memory_order_relaxed);
    }
    return c;
}

template <int D>
void launch_attend(const AttendArgs &aa, int64_t grid, bool direct15, bool spread, hipStream_t s) {
    // direct15: all fifteen head survivors in flight (one block per CU); else eight at a time
    const dim3 g((unsigned)grid), t(kAttendThreads);
    if (direct15) {
        if (spread) hipLaunchKernelGGL((k_attend<D, 15, true>), g, t, 0, s, aa);
        else hipLaunchKernelGGL((k_attend<D, 15, false>), g, t, 0, s, aa);
    } else {
        if (spread) hipLaunchKernelGGL((k_attend<D, 8, true>), g, t, 0, s, aa);
        else hipLaunchKernelGGL((k_attend<D, 8, false>), g, t, 0, s, aa);
    }
}

template <int D, int NT, bool MAT>
void launch_select_t(const SelectArgs &a, int u, int blocks, int threads, hipStream_t s) {
    if (u == 1 || select_tiles<D>() == 1)
        hipLaunchKernelGGL((k_select<D, NT, MAT, 1>), dim3(blocks), dim3(threads), 0, s, a);
    else
        hipLaunchKernelGGL((k_select<D, NT, MAT, select_tiles<D>()>), dim3(blocks), dim3(threads), 0, s, a);
}

template <bool MAT>
void launch_select(const Plan &p, const SelectArgs &a, hipStream_t s) {
    const int blocks = p.B * p.h_k * p.n_chunk;
    // chunks of only kWaves groups (short caches) leave the upper waves
    // without rows: launch the lower four alone
    const int threads = p.chunk_len / p.grp > kWaves ? kSelThreads : kThreads;
    if (p.d == 64) {
        if (p.nt == 1) launch_select_t<64, 1, MAT>(a, p.u, blocks, threads, s);
        else if (p.nt == 2) launch_select_t<64, 2, MAT>(a, p.u, blocks, threads, s);
        else launch_select_t<64, 4, MAT>(a, p.u, blocks, threads, s);
    } else {
        if (p.nt == 1) launch_select_t<128, 1, MAT>(a, p.u, blocks, threads, s);
        else if (p.nt == 2) launch_select_t<128, 2, MAT>(a, p.u, blocks, threads, s);
        else launch_select_t<128, 4, MAT>(a, p.u, blocks, threads, s);
    }
}

SelectArgs select_args(const Plan &p, const void *Q, const void *K, const float *tau, char *ws) {
    SelectArgs a;
    a.Q = (const uint16_t *)Q;
    a.K = (const uint16_t *)K;
    a.tau = tau;
    a.A = (float *)(ws + p.off_scores);
    a.ld_a = p.ld_a;
    a.ld_kv = p.ld_kv;
    a.B = p.B, a.h_q = p.h_q, a.h_k = p.h_k;
    a.n_chunk = p.n_chunk;
    a.l_kv = p.l_kv, a.chunk_len = p.chunk_len;
    a.scale = (float)(1.0 / sqrt((double)p.d));
    a.seg = (int32_t *)(ws + p.off_seg);
    a.n_sub = p.n_sub;
    a.sub_cap = p.sub_cap;
    a.seg_w = p.seg_w;
    a.hist = (uint32_t *)(ws + p.off_hist);
    a.state = (uint32_t *)(ws + p.off_state);
    return a;
}

// Refresh: score pass writing fp32 A, then the exact radix select -> tau.
int run_refresh(const Plan &p, const void *Q, const void *K, float *tau, char *ws,
                hipStream_t s) {
    SelectArgs sa = select_args(p, Q, K, nullptr, ws);
    launch_select<true>(p, sa, s);
    RadixArgs ra;
    ra.A = (const float *)(ws + p.off_scores);
    ra.ld_a = p.ld_a, ra.l_kv = p.l_kv, ra.N = p.N;
    ra.rows = p.rows;
    ra.bpr = p.hist_bpr;
    ra.blk_len = kHistBlock;
    ra.hist = (uint32_t *)(ws + p.off_hist);
    ra.state = (uint32_t *)(ws + p.off_state);
    ra.cand = (uint32_t *)(ws + p.off_cand);
    ra.tau = tau;
    hipLaunchKernelGGL(k_hist, dim3(p.rows * p.hist_bpr), dim3(kThreads), 0, s, ra);
    hipLaunchKernelGGL(k_select1, dim3(p.rows), dim3(kThreads), 0, s, ra);
    hipLaunchKernelGGL(k_collect, dim3(p.rows * p.hist_bpr), dim3(kThreads), 0, s, ra);
    hipLaunchKernelGGL(k_select_final, dim3(p.rows), dim3(kThreads), 0, s, ra);
    return launch_status();
}

int run_attend(const Plan &p, const void *V, float *O, int32_t *counts, char *ws,
               hipStream_t s) {
    AttendArgs aa;
    aa.seg = (const int32_t *)(ws + p.off_seg);
    aa.n_sub = p.n_sub;
    aa.seg_w = p.seg_w;
    aa.sub_cap = (int)p.sub_cap;
    aa.V = (const uint16_t *)V;
    aa.B = p.B, aa.h_q = p.h_q, aa.h_v = p.h_v;
    aa.l_kv = p.l_kv;
    aa.ld_kv = p.ld_kv;
    aa.O = O;
    aa.counts = counts;
    const int64_t grid = attend_grid(p.rows, p.d);
    if (SAGA_ATTEND_ROW && grid >= 2 * (int64_t)device_cus()) {
        // the column split would put two or more blocks on every compute unit: a row per block
        if (p.d == 64)
            hipLaunchKernelGGL(k_attend_row<64>, dim3(p.rows), dim3(kAttendThreads), 0, s, aa);
        else
            hipLaunchKernelGGL(k_attend_row<128>, dim3(p.rows), dim3(kAttendThreads), 0, s, aa);
        return launch_status();
    }
    const bool direct15 = grid <= device_cus();
    const bool spread = p.N > (int64_t)kRecHead * p.n_sub;
    if (p.d == 64)
        launch_attend<64>(aa, grid, direct15, spread, s);
    else
        launch_attend<128>(aa, grid, direct15, spread, s);
    return launch_status();
}

// Selection half of a step: scores, compare with tau (after an exact refresh
// when asked), compaction into the segments and the per-chunk partials.
int run_select(const Plan &p, const void *Q, const void *K, float *tau, int refresh, char *w,
               hipStream_t s) {
    if (refresh) {
        int st = run_refresh(p, Q, K, tau, w, s);
        if (st != SAGA_OK) return st;
        CompactArgs ca;
        ca.A = (const float *)(w + p.off_scores);
        ca.ld_a = p.ld_a, ca.l_kv = p.l_kv, ca.chunk_len = p.chunk_len, ca.grp = p.grp;
        ca.n_chunk = p.n_chunk;
        ca.tau = tau;
        ca.seg = (int32_t *)(w + p.off_seg);
        ca.n_sub = p.n_sub;
        ca.sub_cap = p.sub_cap;
        ca.seg_w = p.seg_w;
        hipLaunchKernelGGL(k_compact, dim3(p.rows * p.n_chunk), dim3(kThreads), 0, s, ca);
    } else {
        SelectArgs sa = select_args(p, Q, K, tau, w);
        launch_select<false>(p, sa, s);
    }
    return launch_status();
}

// k_refine over the current records: the exact N-th largest listed score
// -> tau (and the records' threshold); N positions of the survivors -> pivot.
void launch_refine(const Plan &p, float *tau, int32_t *pivot, char *w, hipStream_t s) {
    RefineArgs r;
    r.seg = (int32_t *)(w + p.off_seg);
    r.n_sub = p.n_sub;
    r.seg_w = p.seg_w, r.sub_cap = p.sub_cap, r.N = p.N;
    r.tau = tau;
    r.pivot = pivot;
    hipLaunchKernelGGL(k_refine, dim3(p.rows), dim3(kThreads), 0, s, r);
}

// Exact refresh from the pivot positions: lower bound per row, a compare
// pass that lists every score at or above it, then k_refine.
int run_pivot_refresh(const Plan &p, const void *Q, const void *K, float *tau, int32_t *pivot,
                      char *w, hipStream_t s) {
    PivotArgs pa;
    pa.Q = (const uint16_t *)Q, pa.K = (const uint16_t *)K;
    pa.B = p.B, pa.h_q = p.h_q, pa.h_k = p.h_k;
    pa.l_kv = p.l_kv, pa.ld_kv = p.ld_kv, pa.N = p.N, pa.chunk_len = p.chunk_len, pa.grp = p.grp;
    pa.scale = (float)(1.0 / sqrt((double)p.d));
    pa.pivot = pivot;
    pa.pi = (float *)(w + p.off_pi);
    if (p.d == 64)
        hipLaunchKernelGGL(k_pivot<64>, dim3(p.rows), dim3(kAttendThreads), 0, s, pa);
    else
        hipLaunchKernelGGL(k_pivot<128>, dim3(p.rows), dim3(kAttendThreads), 0, s, pa);
    SelectArgs sa = select_args(p, Q, K, (const float *)(w + p.off_pi), w);
    launch_select<false>(p, sa, s);
    launch_refine(p, tau, pivot, w, s);
    return launch_status();
}

template <int D, int GMAX, int NV>
void launch_dense_t(const DenseArgs &a, int run, int blocks, hipStream_t s) {
    // a compile-time value-head map for runs of up to 4 query heads per
    // value head that fit the block's head count; else the run-time lookup
    const dim3 g(blocks), t(kThreads);
    if constexpr (NV > 1) {
        if (run == 1) {
            hipLaunchKernelGGL((k_dense<D, GMAX, NV, 1>), g, t, 0, s, a);
            return;
        }
        if constexpr (2 * NV <= GMAX) {
            if (run == 2) {
                hipLaunchKernelGGL((k_dense<D, GMAX, NV, 2>), g, t, 0, s, a);
                return;
            }
        }
        if constexpr (3 * NV <= GMAX) {
            if (run == 3) {
                hipLaunchKernelGGL((k_dense<D, GMAX, NV, 3>), g, t, 0, s, a);
                return;
            }
        }
        if constexpr (4 * NV <= GMAX) {
            if (run == 4) {
                hipLaunchKernelGGL((k_dense<D, GMAX, NV, 4>), g, t, 0, s, a);
                return;
            }
        }
    }
    hipLaunchKernelGGL((k_dense<D, GMAX, NV, 0>), g, t, 0, s, a);
}

template <int D, int NV>
void launch_dense_g(const DensePlan &p, const DenseArgs &a, int blocks, hipStream_t s) {
    if (p.gmax <= 4) launch_dense_t<D, 4, NV>(a, p.run, blocks, s);
    else if (p.gmax <= 8) launch_dense_t<D, 8, NV>(a, p.run, blocks, s);
    else launch_dense_t<D, 16, NV>(a, p.run, blocks, s);
}

// Dense split-KV decode (key heads h_k, value heads h_v) and the merge of
// the chunk partials.
int run_dense(const void *Q, const void *K, const void *V, int B, int h_q, int h_k, int h_v,
              int d, int64_t l_kv, float *O, void *ws, size_t ws_bytes, void *hip_stream) {
    DensePlan p;
    int st = make_dense_plan(B, h_q, h_k, h_v, d, l_kv, &p);
    if (st != SAGA_OK) return st;
    if (!Q || !K || !V || !O || !aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) ||
        !aligned(O, 4))
        return SAGA_ERR_INVALID_ARG;
    if (!ws || !aligned(ws, kAlign)) return SAGA_ERR_INVALID_ARG;
    if (ws_bytes < p.total) return SAGA_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)hip_stream;
    DenseArgs a;
    a.Q = (const uint16_t *)Q, a.K = (const uint16_t *)K, a.V = (const uint16_t *)V;
    a.B = B, a.h_q = h_q, a.h_k = h_k, a.h_v = h_v;
    a.n_chunk = p.n_chunk;
    a.n_vsub = p.n_vsub;
    a.l_kv = l_kv, a.chunk_len = p.chunk_len;
    a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)d));
    a.partial = (float *)ws;
    const int blocks = B * h_k * p.n_vsub * p.n_chunk;
    if (d == 64) {
        if (p.nv == 1) launch_dense_g<64, 1>(p, a, blocks, s);
        else if (p.nv == 2) launch_dense_g<64, 2>(p, a, blocks, s);
        else launch_dense_g<64, 4>(p, a, blocks, s);
    } else {
        if (p.nv == 1) launch_dense_g<128, 1>(p, a, blocks, s);
        else if (p.nv == 2) launch_dense_g<128, 2>(p, a, blocks, s);
        else launch_dense_g<128, 4>(p, a, blocks, s);
    }
    DenseMergeArgs m;
    m.partial = (const float *)ws;
    m.n_chunk = p.n_chunk;
    m.O = O;
    if (d == 64)
        hipLaunchKernelGGL(k_dense_merge<64>, dim3(p.rows), dim3(kThreads), 0, s, m);
    else
        hipLaunchKernelGGL(k_dense_merge<128>, dim3(p.rows), dim3(kThreads), 0, s, m);
    return launch_status();
}

int check_ws(const Plan &p, const void *ws, size_t ws_bytes) {
    if (!ws || !aligned(ws, kAlign)) return SAGA_ERR_INVALID_ARG;
    if (ws_bytes < p.total) return SAGA_ERR_WORKSPACE;
    return SAGA_OK;
}

}  // namespace

extern "C" {

const char *saga_status_string(int status) {
    switch (status) {
        case SAGA_OK: return "SAGA_OK";
        case SAGA_ERR_INVALID_ARG: return "SAGA_ERR_INVALID_ARG";
        case SAGA_ERR_UNSUPPORTED: return "SAGA_ERR_UNSUPPORTED";
        case SAGA_ERR_WORKSPACE: return "SAGA_ERR_WORKSPACE";
        case SAGA_ERR_HIP: return "SAGA_ERR_HIP";
        default: return "SAGA_ERR_UNKNOWN";
    }
}

int saga_version(void) { return 100; }

size_t saga_workspace_bytes(int B, int h_q, int h_k, int h_v, int d, int64_t l_kv, int64_t N) {
    Plan p;
    return make_plan(B, h_q, h_k, h_v, d, l_kv, N, &p) == SAGA_OK ? p.total : 0;
}

size_t saga_dense_workspace_bytes(int B, int h_q, int h_kv, int d, int64_t l_kv) {
    DensePlan p;
    return make_dense_plan(B, h_q, h_kv, h_kv, d, l_kv, &p) == SAGA_OK ? p.total : 0;
}

size_t saga_full_attention_workspace_bytes(int B, int h_q, int h_k, int h_v, int d,
                                           int64_t l_kv) {
    DensePlan p;
    return make_dense_plan(B, h_q, h_k, h_v, d, l_kv, &p) == SAGA_OK ? p.total : 0;
}

int saga_workspace_layout(int B, int h_q, int h_k, int h_v, int d, int64_t l_kv, int64_t N,
                          saga_ws_layout *out) {
    if (!out) return SAGA_ERR_INVALID_ARG;
    Plan p;
    int st = make_plan(B, h_q, h_k, h_v, d, l_kv, N, &p);
    if (st != SAGA_OK) return st;
    out->bytes = p.total;
    out->scores_off = p.off_scores;
    out->scores_ld = p.ld_a;
    out->seg_off = p.off_seg;
    out->seg_words = p.seg_w;
    out->chunk_len = p.chunk_len;
    out->n_chunk = p.n_chunk;
    out->n_seg = p.n_sub;
    out->seg_cap = p.sub_cap;
    out->seg_group = p.grp;
    return SAGA_OK;
}

int saga_workspace_init(void *ws, size_t ws_bytes, void *hip_stream) {
    if (!ws || !aligned(ws, kAlign) || ws_bytes == 0 || ws_bytes % 4) return SAGA_ERR_INVALID_ARG;
    hipStream_t s = (hipStream_t)hip_stream;
    const int64_t n = (int64_t)(ws_bytes / 4);
    int blocks = (int)(ceil_div(n, kThreads) < 4096 ? ceil_div(n, kThreads) : 4096);
    hipLaunchKernelGGL(k_fill_u32, dim3(blocks), dim3(kThreads), 0, s, (uint32_t *)ws, n, 0u);
    return launch_status();
}

int saga_refresh_threshold(const void *Q, const void *K, int B, int h_q, int h_k, int d,
                           int64_t l_kv, int64_t N, float *tau, void *ws, size_t ws_bytes,
                           void *hip_stream) {
    Plan p;
    int st = make_plan(B, h_q, h_k, h_k, d, l_kv, N, &p);
    if (st != SAGA_OK) return st;
    if (!Q || !K || !tau || !aligned(Q, 16) || !aligned(K, 16) || !aligned(tau, 4))
        return SAGA_ERR_INVALID_ARG;
    if ((st = check_ws(p, ws, ws_bytes)) != SAGA_OK) return st;
    return run_refresh(p, Q, K, tau, (char *)ws, (hipStream_t)hip_stream);
}

int saga_select(const void *Q, const void *K, int B, int h_q, int h_k, int h_v, int d,
                int64_t l_kv, int64_t N, float *tau, int refresh, void *ws, size_t ws_bytes,
                void *hip_stream) {
    Plan p;
    int st = make_plan(B, h_q, h_k, h_v, d, l_kv, N, &p);
    if (st != SAGA_OK) return st;
    if (!Q || !K || !tau || !aligned(Q, 16) || !aligned(K, 16) || !aligned(tau, 4))
        return SAGA_ERR_INVALID_ARG;
    if ((st = check_ws(p, ws, ws_bytes)) != SAGA_OK) return st;
    return run_select(p, Q, K, tau, refresh, (char *)ws, (hipStream_t)hip_stream);
}

int saga_attend(const void *V, int B, int h_q, int h_k, int h_v, int d, int64_t l_kv, int64_t N,
                float *O, int32_t *counts, void *ws, size_t ws_bytes, void *hip_stream) {
    Plan p;
    int st = make_plan(B, h_q, h_k, h_v, d, l_kv, N, &p);
    if (st != SAGA_OK) return st;
    if (!V || !O || !aligned(V, 16) || !aligned(O, 4) || (counts && !aligned(counts, 4)))
        return SAGA_ERR_INVALID_ARG;
    if ((st = check_ws(p, ws, ws_bytes)) != SAGA_OK) return st;
    return run_attend(p, V, O, counts, (char *)ws, (hipStream_t)hip_stream);
}

int saga_decode_step(const void *Q, const void *K, const void *V, int B, int h_q, int h_k,
                     int h_v, int d, int64_t l_kv, int64_t N, float *tau, int refresh, float *O,
                     int32_t *counts, void *ws, size_t ws_bytes, void *hip_stream) {
    Plan p;
    int st = make_plan(B, h_q, h_k, h_v, d, l_kv, N, &p);
    if (st != SAGA_OK) return st;
    if (!Q || !K || !V || !tau || !O || !aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) ||
        !aligned(tau, 4) || !aligned(O, 4) || (counts && !aligned(counts, 4)))
        return SAGA_ERR_INVALID_ARG;
    if ((st = check_ws(p, ws, ws_bytes)) != SAGA_OK) return st;
    char *w = (char *)ws;
    hipStream_t s = (hipStream_t)hip_stream;
    if ((st = run_select(p, Q, K, tau, refresh, w, s)) != SAGA_OK) return st;
    return run_attend(p, V, O, counts, w, s);
}

}  // extern "C"

namespace {

// saga_decode_step_pivot / saga_decode_step_cache on a plan.
int decode_pivot(const Plan &p, const void *Q, const void *K, const void *V, float *tau,
                 int32_t *pivot, int refresh, float *O, int32_t *counts, void *ws,
                 size_t ws_bytes, void *hip_stream) {
    int st;
    if (!Q || !K || !V || !tau || !O || !aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) ||
        !aligned(tau, 4) || !aligned(O, 4) || (counts && !aligned(counts, 4)))
        return SAGA_ERR_INVALID_ARG;
    if (refresh < 0 || refresh > 2) return SAGA_ERR_INVALID_ARG;
    if (refresh && (!pivot || !aligned(pivot, 4))) return SAGA_ERR_INVALID_ARG;
    if ((st = check_ws(p, ws, ws_bytes)) != SAGA_OK) return st;
    char *w = (char *)ws;
    hipStream_t s = (hipStream_t)hip_stream;
    if (refresh == 2) {
        st = run_pivot_refresh(p, Q, K, tau, pivot, w, s);
    } else {
        st = run_select(p, Q, K, tau, refresh, w, s);
        if (st == SAGA_OK && refresh == 1) {
            launch_refine(p, tau, pivot, w, s);  // same tau again; records the pivot
            st = launch_status();
        }
    }
    if (st != SAGA_OK) return st;
    return run_attend(p, V, O, counts, w, s);
}

}  // namespace

extern "C" {

int saga_decode_step_pivot(const void *Q, const void *K, const void *V, int B, int h_q, int h_k,
                           int h_v, int d, int64_t l_kv, int64_t N, float *tau, int32_t *pivot,
                           int refresh, float *O, int32_t *counts, void *ws, size_t ws_bytes,
                           void *hip_stream) {
    Plan p;
    int st = make_plan(B, h_q, h_k, h_v, d, l_kv, N, &p);
    if (st != SAGA_OK) return st;
    return decode_pivot(p, Q, K, V, tau, pivot, refresh, O, counts, ws, ws_bytes, hip_stream);
}

size_t saga_cache_workspace_bytes(int B, int h_q, int h_k, int h_v, int d, int64_t cap,
                                  int64_t N) {
    Plan p;
    return make_plan(B, h_q, h_k, h_v, d, cap, N, &p, cap) == SAGA_OK ? p.total : 0;
}

int saga_decode_step_cache(const void *Q, const void *K, const void *V, int B, int h_q, int h_k,
                           int h_v, int d, int64_t cap, int64_t len, int64_t N, float *tau,
                           int32_t *pivot, int refresh, float *O, int32_t *counts, void *ws,
                           size_t ws_bytes, void *hip_stream) {
    Plan p;
    int st = make_plan(B, h_q, h_k, h_v, d, len, N, &p, cap);
    if (st != SAGA_OK) return st;
    return decode_pivot(p, Q, K, V, tau, pivot, refresh, O, counts, ws, ws_bytes, hip_stream);
}

}  // extern "C"

namespace {

// The allocation-free entry point's workspace: one array per GPU, held from the
// library's first use on that GPU until the process ends.  Host code must never
// pass `scratch` itself to a kernel or a copy (in host code the name is a
// host-side stand-in, not the device address): the device address comes from
// hipGetSymbolAddress, once per device, and is kept in scratch_dev[].
constexpr size_t kScratchBytes = size_t(SAGA_STATIC_WORKSPACE_BYTES);
static_assert(kScratchBytes % kAlign == 0, "scratch size");
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void *scratch_dev[kMaxDevices];

// The current device's scratch address (looked up on its first call there).
int scratch_ptr(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SAGA_ERR_HIP;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_dev[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
            (void)hipGetLastError();
            return SAGA_ERR_HIP;
        }
        scratch_dev[dev] = ptr;
    }
    *out = scratch_dev[dev];
    return SAGA_OK;
}

}  // namespace

extern "C" {

int saga_decode_step_noalloc(const void *Q, const void *K, const void *V, int B, int h_q, int h_k,
                             int h_v, int d, int64_t l_kv, int64_t N, float *tau, int32_t *pivot,
                             int refresh, float *O, int32_t *counts, void *hip_stream) {
    Plan p;
    int st = make_plan(B, h_q, h_k, h_v, d, l_kv, N, &p);
    if (st != SAGA_OK) return st;
    if (p.total > kScratchBytes) return SAGA_ERR_WORKSPACE;  // beyond the static workspace
    void *ws = nullptr;
    if ((st = scratch_ptr(&ws)) != SAGA_OK) return st;
    return decode_pivot(p, Q, K, V, tau, pivot, refresh, O, counts, ws, kScratchBytes, hip_stream);
}

int saga_append_kv(void *K, void *V, const void *k_new, const void *v_new, int B, int h_k,
                   int h_v, int d, int64_t cap, int64_t pos, void *hip_stream) {
    if (B < 1 || h_k < 1 || h_v < h_k || cap < 1 || pos < 0 || pos >= cap)
        return SAGA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return SAGA_ERR_UNSUPPORTED;
    if (cap * (int64_t)d * 2 >= (int64_t(1) << 31)) return SAGA_ERR_UNSUPPORTED;
    if (!K || !V || !k_new || !v_new || !aligned(K, 16) || !aligned(V, 16) ||
        !aligned(k_new, 16) || !aligned(v_new, 16))
        return SAGA_ERR_INVALID_ARG;
    AppendArgs a;
    a.K = (uint16_t *)K, a.V = (uint16_t *)V;
    a.k_new = (const uint16_t *)k_new, a.v_new = (const uint16_t *)v_new;
    a.B = B, a.h_k = h_k, a.h_v = h_v, a.d = d;
    a.ld_kv = cap, a.pos = pos;
    const int64_t pieces = (int64_t)B * (h_k + h_v) * (d / 8);
    const int blocks = (int)std::min<int64_t>(ceil_div(pieces, kThreads), 1024);
    hipLaunchKernelGGL(k_append, dim3(blocks), dim3(kThreads), 0, (hipStream_t)hip_stream, a);
    return launch_status();
}

int saga_dense_gqa_baseline(const void *Q, const void *K, const void *V, int B, int h_q,
                            int h_kv, int d, int64_t l_kv, float *O, void *ws, size_t ws_bytes,
                            void *hip_stream) {
    return run_dense(Q, K, V, B, h_q, h_kv, h_kv, d, l_kv, O, ws, ws_bytes, hip_stream);
}

int saga_full_attention(const void *Q, const void *K, const void *V, int B, int h_q, int h_k,
                        int h_v, int d, int64_t l_kv, float *O, void *ws, size_t ws_bytes,
                        void *hip_stream) {
    return run_dense(Q, K, V, B, h_q, h_k, h_v, d, l_kv, O, ws, ws_bytes, hip_stream);
}

int saga_selection_mask(const void *ws, size_t ws_bytes, int B, int h_q, int h_k, int h_v, int d,
                        int64_t l_kv, int64_t N, uint8_t *mask, void *hip_stream) {
    Plan p;
    int st = make_plan(B, h_q, h_k, h_v, d, l_kv, N, &p);
    if (st != SAGA_OK) return st;
    if (!mask) return SAGA_ERR_INVALID_ARG;
    if ((st = check_ws(p, ws, ws_bytes)) != SAGA_OK) return st;
    hipStream_t s = (hipStream_t)hip_stream;
    const char *w = (const char *)ws;
    const int64_t n = (int64_t)p.rows * l_kv;
    int blocks = (int)(ceil_div(n, kThreads) < 4096 ? ceil_div(n, kThreads) : 4096);
    hipLaunchKernelGGL(k_fill_u8, dim3(blocks), dim3(kThreads), 0, s, mask, n, (uint8_t)0);
    MaskArgs ma;
    ma.seg = (const int32_t *)(w + p.off_seg);
    ma.n_sub = p.n_sub;
    ma.sub_cap = p.sub_cap;
    ma.seg_w = p.seg_w;
    ma.l_kv = l_kv;
    ma.mask = mask;
    hipLaunchKernelGGL(k_mask, dim3(p.rows * p.n_sub), dim3(kThreads), 0, s, ma);
    return launch_status();
}

}  // extern "C"

namespace {

template <int W, int U>
void launch_probe_shape(const void *buf, int64_t n16, int blocks, bool chunked, uint32_t *sink,
                        hipStream_t s) {
    const int64_t per = ceil_div(n16, blocks);
    if (chunked)
        hipLaunchKernelGGL((k_read_probe_shape<W, U, true>), dim3(blocks), dim3(W * kWave), 0, s,
                           (const u32x4 *)buf, n16, per, sink, SAGA_PROBE_SINK_WORDS);
    else
        hipLaunchKernelGGL((k_read_probe_shape<W, U, false>), dim3(blocks), dim3(W * kWave), 0, s,
                           (const u32x4 *)buf, n16, per, sink, SAGA_PROBE_SINK_WORDS);
}

}  // namespace

extern "C" {

int saga_read_probe_shape(const void *buf, int64_t bytes, int blocks, int waves, int loads,
                          int chunked, uint32_t *sink, void *hip_stream) {
    if (!buf || !sink || !aligned(buf, 16) || !aligned(sink, 4) || bytes <= 0 || bytes % 16 != 0)
        return SAGA_ERR_INVALID_ARG;
    if (blocks < 1 || blocks > 65536) return SAGA_ERR_INVALID_ARG;
    const int64_t n16 = bytes / 16;
    hipStream_t s = (hipStream_t)hip_stream;
    const bool ch = chunked != 0;
    if (waves == 4 && loads == 4) launch_probe_shape<4, 4>(buf, n16, blocks, ch, sink, s);
    else if (waves == 4 && loads == 8) launch_probe_shape<4, 8>(buf, n16, blocks, ch, sink, s);
    else if (waves == 4 && loads == 16) launch_probe_shape<4, 16>(buf, n16, blocks, ch, sink, s);
    else if (waves == 8 && loads == 4) launch_probe_shape<8, 4>(buf, n16, blocks, ch, sink, s);
    else if (waves == 8 && loads == 8) launch_probe_shape<8, 8>(buf, n16, blocks, ch, sink, s);
    else return SAGA_ERR_UNSUPPORTED;
    return launch_status();
}

int saga_read_probe(const void *buf, int64_t bytes, uint32_t *sink, void *hip_stream) {
    if (!buf || !sink || !aligned(buf, 16) || !aligned(sink, 4) || bytes <= 0 || bytes % 16 != 0)
        return SAGA_ERR_INVALID_ARG;
    const int64_t n16 = bytes / 16;
    static_assert(kTargetSelectBlocks <= SAGA_PROBE_SINK_WORDS, "probe sink");
    const int64_t per = ceil_div(n16, kTargetSelectBlocks);
    const int blocks = (int)ceil_div(n16, per);
    hipLaunchKernelGGL(k_read_probe, dim3(blocks), dim3(kSelThreads), 0, (hipStream_t)hip_stream,
                       (const u32x4 *)buf, n16, per, sink);
    return launch_status();
}

}  // extern "C"
