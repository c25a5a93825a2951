// merge.hip -- host side of the GQA -> SAGA key-head merge (C ABI in include/saga_merge.h).
//
// Launch sequence on one stream:
//   k_kproj<BM>      K = X W_K^T                                  (n/BM x h_kt*d/128 blocks)
//   k_gram<D,1>      per-chunk second moments S_r of each group's queries (h_kt items)
//   k_gram<D,0>      per-chunk second moments G_p of K_a - K_b         (one item per pair)
//   k_gram_reduce    fixed-order fp64 sum over chunks
//   k_pair_inv<D>    S^-1 by blocked sweeps when S = S_a + S_b is comfortably full rank
//   k_pair_pinv<D>   S^+ by pivoted Cholesky for the other pairs            (one block per pair)
//   k_pair_maps<D>   P_a = S_a S^+, P_b = S_b S^+               (pairs x tile groups)
//   k_pair_cost<D>   partial eq. 13 costs                          (pairs x tile groups)
//   k_match          pair costs from the partials, then the minimum-weight perfect
//                    matching                                          (one block)
//   k_merged_weight  eq. 15 in the weight layout     (h_kt/2 x d/16 x d_model/64 blocks)
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include <algorithm>

#include "../../include/saga_merge.h"
#include "merge_kernels.hpp"

namespace {

using namespace saga::merge;

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

constexpr int64_t kGramBlockBudget = 32768;   // Gram blocks per launch times d
constexpr int64_t kMinGramBlocks = 128;

// tile groups per pair in the map and cost kernels (2 (d/16)^2 tiles, 4 per block)
int cost_parts(int d) { return 2 * (d / 16) * (d / 16) / kTilesPerBlock; }

struct MergePlan {
    int64_t n;
    int h_q, h_kt, d, dm, P, items, nq, nd;
    int64_t ct_q, ct_d;   // tokens per Gram block: query items, key-difference items
    int64_t ldt;          // tokens of the projected keys (n rounded up to 128; kfrag_index)
    size_t off_K, off_part, off_SG, off_Sp, off_Pm, off_cost, off_rank, off_dp, off_choice,
        bytes;
};

int make_merge_plan(int64_t n, int h_q, int h_kt, int d, int d_model, MergePlan *p) {
    if (n < 1 || h_q < 1 || h_kt < 1 || d < 1 || d_model < 1) return SAGA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return SAGA_ERR_UNSUPPORTED;
    if (h_kt % 2 || h_kt < 2 || h_kt > kMaxHeads) return SAGA_ERR_UNSUPPORTED;
    if (h_q < h_kt || h_q > 1024) return SAGA_ERR_UNSUPPORTED;
    if (d_model % 64 || d_model < 64 || d_model > 32768) return SAGA_ERR_UNSUPPORTED;
    if (n > ((int64_t)1 << 26)) return SAGA_ERR_UNSUPPORTED;
    p->n = n;
    p->h_q = h_q;
    p->h_kt = h_kt;
    p->d = d;
    p->dm = d_model;
    p->P = h_kt * (h_kt - 1) / 2;
    p->items = h_kt + p->P;
    // Samples per Gram block, per launch (measured on both layer shapes): about
    // kGramBlockBudget / d blocks -- a d x d partial costs d^2 words to write and
    // reduce -- with at least 4 d samples per query block; key-difference blocks
    // take at least 16 d samples unless that leaves fewer than kMinGramBlocks
    // blocks, and then at least 256 (4 d at d = 64; 2 d at d = 128, whose tile
    // groups split a chunk four ways).
    const int64_t g_max = ceil_div(h_q, h_kt);
    const int64_t target = kGramBlockBudget / d;
    const int64_t s_q = std::max<int64_t>(4 * d, ceil_div(n * h_q, target));
    int64_t s_d = std::max<int64_t>(16 * d, ceil_div(n * p->P, target));
    if (p->P * ceil_div(n, s_d) < kMinGramBlocks)
        s_d = std::max<int64_t>(256, ceil_div(n * p->P, kMinGramBlocks));
    p->ct_q = ceil_div(s_q, g_max);
    p->ct_d = ceil_div(s_d, kPBM) * kPBM;   // four waves x whole 32-token MFMA steps
    p->ldt = ceil_div(n, kPBM) * kPBM;
    p->nq = (int)ceil_div(n, p->ct_q);
    p->nd = (int)ceil_div(p->ldt, p->ct_d);
    const size_t dd = (size_t)d * d * sizeof(float);
    size_t o = 0;
    p->off_K = o;      o = align_up(o + (size_t)p->ldt * h_kt * d * sizeof(float));
    p->off_part = o;   o = align_up(o + ((size_t)h_kt * p->nq + (size_t)p->P * p->nd) * dd);
    p->off_SG = o;     o = align_up(o + (size_t)p->items * dd);
    p->off_Sp = o;     o = align_up(o + (size_t)p->P * dd);
    p->off_Pm = o;     o = align_up(o + (size_t)p->P * 2 * dd);
    p->off_cost = o;   o = align_up(o + (size_t)p->P * cost_parts(d) * sizeof(double));
    p->off_rank = o;   o = align_up(o + (size_t)p->P * sizeof(int));
    p->off_dp = o;     o = align_up(o + ((size_t)1 << h_kt) * sizeof(double));
    p->off_choice = o; o = align_up(o + ((size_t)1 << h_kt));
    p->bytes = o;
    return SAGA_OK;
}

bool aligned(const void *ptr, size_t a) { return ((uintptr_t)ptr % a) == 0; }

void pair_table(int h_kt, uint8_t *pa, uint8_t *pb) {
    int p = 0;
    for (int a = 0; a < h_kt; ++a)
        for (int b = a + 1; b < h_kt; ++b, ++p) {
            pa[p] = (uint8_t)a;
            pb[p] = (uint8_t)b;
        }
}

// dynamic LDS of k_pair_pinv (two padded d x d matrices and two pivot rows) and
// of k_pair_inv
size_t pinv_lds_bytes(int d) {
    return ((size_t)2 * d * (d + 4) + (size_t)2 * d) * sizeof(float);
}
size_t inv_lds_bytes(int d) { return (size_t)blocked_lds_floats(d) * sizeof(float); }

// The d = 128 pseudoinverse and the projection's LDS rings take more than
// 64 KB of dynamic LDS; say so once per process.
int lds_limits_once() {
    static int status = [] {
        const hipFuncAttribute at = hipFuncAttributeMaxDynamicSharedMemorySize;
        const bool ok =
            hipFuncSetAttribute((const void *)k_pair_pinv<128>, at, (int)pinv_lds_bytes(128)) ==
                hipSuccess &&
            hipFuncSetAttribute((const void *)k_pair_inv<128>, at, (int)inv_lds_bytes(128)) ==
                hipSuccess &&
            hipFuncSetAttribute((const void *)k_kproj<128>, at, (int)proj_lds_bytes(128)) ==
                hipSuccess &&
            hipFuncSetAttribute((const void *)k_kproj<256>, at, (int)proj_lds_bytes(256)) ==
                hipSuccess;
        return ok ? (int)SAGA_OK : (int)SAGA_ERR_HIP;
    }();
    return status;
}

// Projection tile height: 256 tokens when that still gives a block per compute
// unit (256 blocks), else 128.
template <int BM>
void launch_kproj(const ProjArgs &pa, hipStream_t s) {
    hipLaunchKernelGGL(k_kproj<BM>, dim3((unsigned)ceil_div(pa.n, BM), (unsigned)(pa.cols / kPBN)),
                       dim3(proj_threads(BM)), proj_lds_bytes(BM), s, pa);
}

template <int D>
int run_merge(const MergePlan &p, const void *X, const void *Q, const void *W_K,
              const int32_t *pairs_in, float *W_merged, int32_t *pairs, double *pair_loss,
              double *total_loss, char *ws, hipStream_t s) {
    float *K = (float *)(ws + p.off_K);
    float *part = (float *)(ws + p.off_part);
    float *SG = (float *)(ws + p.off_SG);
    float *Sp = (float *)(ws + p.off_Sp);
    float *Pm = (float *)(ws + p.off_Pm);

    ProjArgs pa{(const uint16_t *)X, (const uint16_t *)W_K, K, p.n, p.ldt, p.dm, p.h_kt * D};
    if (ceil_div(p.n, 256) * (p.h_kt * D / kPBN) >= 256) launch_kproj<256>(pa, s);
    else launch_kproj<128>(pa, s);

    GramArgs ga{};
    ga.Q = (const uint16_t *)Q;
    ga.Kt = K;
    ga.ldt = p.ldt;
    ga.n = p.n;
    ga.h_q = p.h_q;
    ga.h_kt = p.h_kt;
    pair_table(p.h_kt, ga.pa, ga.pb);
    ga.part = part;
    ga.chunk_tokens = p.ct_q;
    ga.n_chunk = p.nq;
    hipLaunchKernelGGL((k_gram<D, true>), dim3((unsigned)p.nq, (unsigned)p.h_kt, gram_groups(D, true)),
                       dim3(kThreads), 0, s, ga);
    ga.part = part + (size_t)p.h_kt * p.nq * D * D;
    ga.chunk_tokens = p.ct_d;
    ga.n_chunk = p.nd;
    hipLaunchKernelGGL((k_gram<D, false>), dim3((unsigned)p.nd, (unsigned)p.P, gram_groups(D, false)),
                       dim3(kThreads), 0, s, ga);

    ReduceArgs ra{part, SG, p.h_kt, p.nq, p.nd, D * D};
    hipLaunchKernelGGL(k_gram_reduce, dim3((unsigned)ceil_div(D * D, kThreads), (unsigned)p.items),
                       dim3(kThreads), 0, s, ra);

    PinvArgs ia{};
    ia.SG = SG;
    ia.Sp = Sp;
    ia.rank = (int *)(ws + p.off_rank);
    ia.h_kt = p.h_kt;
    pair_table(p.h_kt, ia.pa, ia.pb);
    hipLaunchKernelGGL(k_pair_inv<D>, dim3((unsigned)p.P), dim3(pinv_threads(D)), inv_lds_bytes(D), s,
                       ia);
    hipLaunchKernelGGL(k_pair_pinv<D>, dim3((unsigned)p.P), dim3(pinv_threads(D)), pinv_lds_bytes(D), s,
                       ia);

    LossArgs la{};
    la.SG = SG;
    la.Sp = Sp;
    la.Pm = Pm;
    la.part = (double *)(ws + p.off_cost);
    la.h_kt = p.h_kt;
    la.n_part = cost_parts(D);
    pair_table(p.h_kt, la.pa, la.pb);
    hipLaunchKernelGGL(k_pair_maps<D>, dim3((unsigned)p.P, (unsigned)cost_parts(D)), dim3(kThreads),
                       0, s, la);
    hipLaunchKernelGGL(k_pair_cost<D>, dim3((unsigned)p.P, (unsigned)cost_parts(D)), dim3(kThreads),
                       0, s, la);

    MatchArgs ma{};
    ma.part = (const double *)(ws + p.off_cost);
    ma.n_part = cost_parts(D);
    ma.w = pair_loss;
    ma.dp = (double *)(ws + p.off_dp);
    ma.choice = (uint8_t *)(ws + p.off_choice);
    ma.pairs = pairs;
    ma.total = total_loss;
    ma.h_kt = p.h_kt;
    ma.forced = pairs_in != nullptr;
    if (pairs_in) {
        // canonical order: a < b within a pair, pairs sorted by a
        int a_of[kMaxHeads / 2], b_of[kMaxHeads / 2];
        for (int i = 0; i < p.h_kt / 2; ++i) {
            const int x = pairs_in[2 * i], y = pairs_in[2 * i + 1];
            a_of[i] = x < y ? x : y;
            b_of[i] = x < y ? y : x;
        }
        for (int i = 0; i < p.h_kt / 2; ++i)
            for (int j = i + 1; j < p.h_kt / 2; ++j)
                if (a_of[j] < a_of[i]) {
                    int t = a_of[i]; a_of[i] = a_of[j]; a_of[j] = t;
                    t = b_of[i]; b_of[i] = b_of[j]; b_of[j] = t;
                }
        for (int i = 0; i < p.h_kt / 2; ++i) {
            ma.fa[i] = (uint8_t)a_of[i];
            ma.fb[i] = (uint8_t)b_of[i];
        }
    }
    hipLaunchKernelGGL(k_match, dim3(1), dim3(kThreads), 0, s, ma);

    WeightArgs wa{(const uint16_t *)W_K, Pm, pairs, W_merged, p.dm, p.h_kt};
    hipLaunchKernelGGL(k_merged_weight<D>,
                       dim3((unsigned)(p.h_kt / 2), (unsigned)(D / kWC), (unsigned)(p.dm / kWX)),
                       dim3(kThreads), 0, s, wa);
    return hipGetLastError() == hipSuccess ? SAGA_OK : SAGA_ERR_HIP;
}

}  // namespace

extern "C" {

size_t saga_merge_workspace_bytes(int64_t n, int h_q, int h_kt, int d, int d_model) {
    MergePlan p;
    return make_merge_plan(n, h_q, h_kt, d, d_model, &p) == SAGA_OK ? p.bytes : 0;
}

int saga_merge_key_heads(const void *X, const void *Q, const void *W_K, int64_t n, int h_q,
                         int h_kt, int d, int d_model, const int32_t *pairs_in, float *W_merged,
                         int32_t *pairs, double *pair_loss, double *total_loss, void *ws,
                         size_t ws_bytes, void *hip_stream) {
    MergePlan p;
    const int st = make_merge_plan(n, h_q, h_kt, d, d_model, &p);
    if (st != SAGA_OK) return st;
    const void *ptrs16[] = {X, Q, W_K, W_merged, pair_loss, total_loss, ws};
    for (const void *ptr : ptrs16)
        if (!ptr || !aligned(ptr, 16)) return SAGA_ERR_INVALID_ARG;
    if (!pairs || !aligned(pairs, 4)) return SAGA_ERR_INVALID_ARG;
    if (pairs_in) {
        int seen[kMaxHeads] = {0};
        for (int i = 0; i < h_kt; ++i) {
            const int x = pairs_in[i];
            if (x < 0 || x >= h_kt || seen[x]) return SAGA_ERR_INVALID_ARG;
            seen[x] = 1;
        }
    }
    if (ws_bytes < p.bytes) return SAGA_ERR_WORKSPACE;
    if (lds_limits_once() != SAGA_OK) return SAGA_ERR_HIP;
    hipStream_t s = (hipStream_t)hip_stream;
    char *w = (char *)ws;
    return d == 64 ? run_merge<64>(p, X, Q, W_K, pairs_in, W_merged, pairs, pair_loss, total_loss,
                                   w, s)
                   : run_merge<128>(p, X, Q, W_K, pairs_in, W_merged, pairs, pair_loss,
                                    total_loss, w, s);
}

}  // extern "C"
