// merge_kernels.hpp -- kernels of the GQA -> SAGA key-head merge (gfx950 / CDNA4).
//
// Method ("More Value per Key", picx.dev summary, GQA-to-SAGA Conversion,
// Stage 1): teacher key heads are merged in pairs (a, b); the merged key
// projection is eq. 15, (W_a S_a + W_b S_b)(S_a + S_b)^+ with S_r the summed
// second moment of group r's calibration queries; a pair's cost is eq. 13 at
// that projection; the pairing minimises eq. 14, i.e. (Theorem 4.2) it is a
// minimum-weight perfect matching on those costs.
//
// How the kernels get there without ever forming an n x n logit matrix:
// with K_r = X W_r the teacher keys, D = K_a - K_b, G = D^T D,
// S = S_a + S_b, P_a = S_a S^+ and P_b = S_b S^+,
//     eq. 13 at eq. 15 = <G P_b, P_b S_a> + <G P_a, P_a S_b>
// (the part of the merged key outside range(S) is annihilated by S_a and S_b,
// so the identity holds for singular S too).  So the data-parallel work is
//   1. the key projection K = X W^T               (bf16 MFMA GEMM, fp32 out),
//   2. d x d Gram matrices over the calibration tokens: S_r for every group
//      and G for every head pair                  (fp32 MFMA, exact products),
// and the rest is small dense algebra per head pair (an eigendecomposition
// for the pseudoinverse, a handful of d x d products) plus a 2^h_kt-state
// matching.
#pragma once

#include "saga_device.hpp"

namespace saga {
namespace merge {

constexpr int kThreads = 256;
constexpr int kMaxHeads = 16;                       // teacher key heads (h_kt)
constexpr int kMaxPairs = kMaxHeads * (kMaxHeads - 1) / 2;
constexpr float kEigRtol = 6.103515625e-05f;        // 2^-14: eigenvalues <= this * max are zero
constexpr int kMaxSweeps = 16;

typedef float f32x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4v mfma4(float a, float b, f32x4v c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// ------------------------------------------------------------------ 1. keys

struct ProjArgs {
    const uint16_t *X;  // [n][dm] bf16
    const uint16_t *W;  // [cols][dm] bf16 (row r*D + c = channel c of teacher key head r)
    float *K;           // [n][cols] fp32
    int64_t n;
    int dm;
    int cols;
};

constexpr int kPBM = 128, kPBN = 128, kPBK = 64;    // block tile (tokens x columns x k)

// LDS tile [128 rows][64 k] bf16: row = 8 chunks of 16 B, chunk c of row r stored
// at chunk position c ^ (r & 7), so the 16 rows one MFMA operand read touches
// fall on different banks.
__device__ __forceinline__ int swz(int row, int chunk) { return row * 8 + (chunk ^ (row & 7)); }

// K = X W^T.  256 threads = 2 x 2 waves, each wave a 64 x 64 sub-tile of 4 x 4
// MFMA 16x16x32 tiles; X and W tiles pass through LDS, double-buffered.
__global__ __launch_bounds__(kThreads) void k_kproj(ProjArgs a) {
    __shared__ u32x4 As[2][kPBM * 8];
    __shared__ u32x4 Bs[2][kPBN * 8];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t t0 = (int64_t)blockIdx.x * kPBM;
    const int n0 = blockIdx.y * kPBN;
    const int lr = tid >> 3, lc = tid & 7;          // load mapping: row lr + 32 i, chunk lc
    const int64_t last = a.n - 1;

    const uint16_t *xrow[4], *wrow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int64_t t = t0 + lr + 32 * i;
        t = t < last ? t : last;
        xrow[i] = a.X + t * a.dm + lc * 8;
        wrow[i] = a.W + (int64_t)(n0 + lr + 32 * i) * a.dm + lc * 8;
    }
    f32x4v acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4v{0.f, 0.f, 0.f, 0.f};

    u32x4 xa[4], wb[4];
    auto gload = [&](int kt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            xa[i] = ld16(xrow[i] + kt * kPBK);
            wb[i] = ld16(wrow[i] + kt * kPBK);
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            As[buf][swz(lr + 32 * i, lc)] = xa[i];
            Bs[buf][swz(lr + 32 * i, lc)] = wb[i];
        }
    };
    const int nk = a.dm / kPBK;
    gload(0);
    lstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
        for (int s = 0; s < 2; ++s) {               // two k-steps of 32 per tile
            const int ch = s * 4 + (lane >> 4);
            bf16x8 af[4], bfr[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                af[i] = as_bf16x8(As[cur][swz(wm * 64 + i * 16 + (lane & 15), ch)]);
                bfr[i] = as_bf16x8(Bs[cur][swz(wn * 64 + i * 16 + (lane & 15), ch)]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j],
                                                                        0, 0, 0);
        }
        if (kt + 1 < nk) lstore(cur ^ 1);
        __syncthreads();
    }
    // lane holds rows 4*(lane/16)+r, column lane%16 of each 16 x 16 tile
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t t = t0 + wm * 64 + i * 16 + (lane >> 4) * 4 + r;
            if (t < a.n) {
                float *row = a.K + t * a.cols + n0 + wn * 64 + (lane & 15);
#pragma unroll
                for (int j = 0; j < 4; ++j) row[j * 16] = acc[i][j][r];
            }
        }
}

// ------------------------------------------------------------ 2. Grams

struct GramArgs {
    const uint16_t *Q;   // [n][h_q][D] bf16 calibration queries
    const float *K;      // [n][h_kt*D] fp32 projected keys
    float *part;         // [items][n_chunk][D][D] per-block partial sums
    int64_t n;
    int64_t chunk_tokens;
    int n_chunk;
    int h_q, h_kt;
    uint8_t pa[kMaxPairs], pb[kMaxPairs];  // pair p = (pa[p], pb[p]), pa < pb
};

// Channel held by row/column i (0..15) of feature block I: lane (k, i) loads
// the float4 at channels 64h + 4i .. 4i+3 of its sample, and register c of that
// chunk feeds block I = 4h + c.  The Gram is accumulated in this permuted
// channel order and un-permuted when written out.
__device__ __forceinline__ int chan(int I, int i) { return 64 * (I >> 2) + 4 * i + (I & 3); }

// One block per (item, token chunk).  Items 0..h_kt-1: S_r, the second moment of
// group r's query vectors (samples = (token, query head of the group)).  Items
// h_kt..: G_p for pair p, the second moment of K_a - K_b (samples = tokens).
// MFMA 16x16x4 fp32: lane (k = lane/16, i = lane%16) supplies sample k's channel
// chan(I, i) as both the A (row) and B (column) operand, so each instruction adds
// 4 samples' outer products to a 16 x 16 tile; only tiles I <= J are formed.
template <int D>
__global__ __launch_bounds__(kThreads) void k_gram(GramArgs a) {
    constexpr int NB = D / 16;                     // feature blocks
    constexpr int NT = NB * (NB + 1) / 2;          // tiles I <= J
    constexpr int NH = D / 64;                     // float4 chunks per lane per sample
    __shared__ float red[D * D];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int k = lane >> 4, i = lane & 15;
    const int item = blockIdx.y;
    const bool is_q = item < a.h_kt;
    const int64_t t_beg = (int64_t)blockIdx.x * a.chunk_tokens;
    int64_t t_end = t_beg + a.chunk_tokens;
    t_end = t_end < a.n ? t_end : a.n;
    const int64_t ntok = t_end > t_beg ? t_end - t_beg : 0;

    int lo = 0, g = 1, ka = 0, kb = 0;
    if (is_q) {
        lo = (item * a.h_q + a.h_kt - 1) / a.h_kt;                 // first j with j*h_kt/h_q >= item
        const int hi = ((item + 1) * a.h_q + a.h_kt - 1) / a.h_kt;
        g = hi - lo;
    } else {
        ka = a.pa[item - a.h_kt];
        kb = a.pb[item - a.h_kt];
    }
    const int64_t n_samp = ntok * g;
    const int64_t per_wave = ((n_samp + 15) / 16) * 4;             // multiple of 4
    const int64_t s_beg = wave * per_wave;
    int64_t s_end = s_beg + per_wave;
    s_end = s_end < n_samp ? s_end : n_samp;
    const int64_t ldk = (int64_t)a.h_kt * D;

    f32x4v acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x4v{0.f, 0.f, 0.f, 0.f};

    for (int64_t s0 = s_beg; s0 < s_end; s0 += 4) {
        const int64_t s = s0 + k;
        const bool ok = s < s_end;
        const int64_t sc = ok ? s : s_beg;
        float x[NB];
        if (is_q) {
            const int64_t t = t_beg + sc / g;
            const int j = lo + (int)(sc % g);
            const uint16_t *src = a.Q + (t * a.h_q + j) * D + 4 * i;
#pragma unroll
            for (int h = 0; h < NH; ++h) {
                const uint2 w = *(const uint2 *)(src + 64 * h);
                x[4 * h + 0] = bf_lo(w.x);
                x[4 * h + 1] = bf_hi(w.x);
                x[4 * h + 2] = bf_lo(w.y);
                x[4 * h + 3] = bf_hi(w.y);
            }
        } else {
            const float *src = a.K + (t_beg + sc) * ldk + 4 * i;
#pragma unroll
            for (int h = 0; h < NH; ++h) {
                const float4 u = *(const float4 *)(src + ka * D + 64 * h);
                const float4 v = *(const float4 *)(src + kb * D + 64 * h);
                x[4 * h + 0] = u.x - v.x;
                x[4 * h + 1] = u.y - v.y;
                x[4 * h + 2] = u.z - v.z;
                x[4 * h + 3] = u.w - v.w;
            }
        }
        if (!ok) {
#pragma unroll
            for (int I = 0; I < NB; ++I) x[I] = 0.f;
        }
#pragma unroll
        for (int I = 0; I < NB; ++I)
#pragma unroll
            for (int J = I; J < NB; ++J) {
                const int t = I * NB - I * (I - 1) / 2 + (J - I);   // tile index of (I, J)
                acc[t] = mfma4(x[I], x[J], acc[t]);
            }
    }

    // Sum the four waves' tiles into LDS one wave at a time, mirroring I < J tiles.
    for (int w = 0; w < 4; ++w) {
        if (wave == w) {
            int t = 0;
#pragma unroll
            for (int I = 0; I < NB; ++I)
#pragma unroll
                for (int J = I; J < NB; ++J, ++t)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int row = chan(I, 4 * k + r), col = chan(J, i);
                        const float v = acc[t][r];
                        if (w == 0) {
                            red[row * D + col] = v;
                            if (I != J) red[col * D + row] = v;
                        } else {
                            red[row * D + col] += v;
                            if (I != J) red[col * D + row] += v;
                        }
                    }
        }
        __syncthreads();
    }
    float *dst = a.part + ((int64_t)item * a.n_chunk + blockIdx.x) * (D * D);
    for (int e = tid; e < D * D; e += kThreads) dst[e] = red[e];
}

struct ReduceArgs {
    const float *part;   // [items][n_chunk][D*D]
    float *out;          // [items][D*D]
    int n_chunk;
    int dd;              // D*D
};

// Fixed-order fp64 sum of the per-block partials (deterministic).
__global__ __launch_bounds__(kThreads) void k_gram_reduce(ReduceArgs a) {
    const int e = blockIdx.x * kThreads + threadIdx.x;
    if (e >= a.dd) return;
    const int item = blockIdx.y;
    const float *p = a.part + (int64_t)item * a.n_chunk * a.dd + e;
    double s = 0.0;
    for (int c = 0; c < a.n_chunk; ++c) s += (double)p[(int64_t)c * a.dd];
    a.out[(int64_t)item * a.dd + e] = (float)s;
}

// --------------------------------------------- 3. eigendecomposition per pair

struct EigArgs {
    const float *SG;     // [h_kt + P][D][D]: S_r, then G_p
    float *V;            // [P][D][D] eigenvectors (column i = vector i)
    float *lam;          // [P][D]
    int h_kt;
    uint8_t pa[kMaxPairs], pb[kMaxPairs];
};

// Partner slots of the round-robin (circle) schedule: in round k of a sweep the
// D indices are split into D/2 disjoint pairs (slot(k, m), slot(k, D-1-m));
// over D-1 rounds every pair of indices meets once.
__device__ __forceinline__ int rr_slot(int k, int m, int D) {
    return m == 0 ? 0 : 1 + (m - 1 + k) % (D - 1);
}

// Cyclic Jacobi eigenvalue method (two-sided rotations, parallel round-robin
// ordering) on S = S_a + S_b, one block per pair, A and V in LDS with rows
// padded to D+1 words (row and column sweeps then hit distinct banks).  A
// rotation is skipped when |a_pq| is at rounding level relative to the
// geometric mean of its diagonal pair (or to ||S||_F); the sweeps stop when a
// whole sweep rotates nothing.
template <int D>
__global__ __launch_bounds__(kThreads) void k_pair_eig(EigArgs a) {
    constexpr int LD = D + 1;
    constexpr int H = D / 2;
    extern __shared__ float sm[];
    float *A = sm;
    float *V = sm + D * LD;
    float *rc = V + D * LD;          // [H] cos
    float *rs = rc + H;              // [H] sin
    int *rp = (int *)(rs + H);       // [H]
    int *rq = rp + H;                // [H]
    int *flag = rq + H;              // [1]
    float *wsum = (float *)(flag + 1);   // [4]
    const int tid = threadIdx.x;
    const int p = blockIdx.x;
    const float *Sa = a.SG + (int64_t)a.pa[p] * D * D;
    const float *Sb = a.SG + (int64_t)a.pb[p] * D * D;

    float fro = 0.f;
    for (int e = tid; e < D * D; e += kThreads) {
        const int r = e / D, c = e % D;
        const float v = 0.5f * ((Sa[r * D + c] + Sb[r * D + c]) + (Sa[c * D + r] + Sb[c * D + r]));
        A[r * LD + c] = v;
        V[r * LD + c] = (r == c) ? 1.f : 0.f;
        fro += v * v;
    }
    fro = wave_sum(fro);
    if ((tid & 63) == 0) wsum[tid >> 6] = fro;
    __syncthreads();
    fro = sqrtf(wsum[0] + wsum[1] + wsum[2] + wsum[3]);
    const float abs_floor = 1.4901161193847656e-08f * fro;   // 2^-26 ||S||_F

    for (int sweep = 0; sweep < kMaxSweeps; ++sweep) {
        if (tid == 0) *flag = 0;
        __syncthreads();
        for (int k = 0; k < D - 1; ++k) {
            if (tid < H) {
                int pp = rr_slot(k, tid, D), qq = rr_slot(k, D - 1 - tid, D);
                if (pp > qq) { const int x = pp; pp = qq; qq = x; }
                const float app = A[pp * LD + pp], aqq = A[qq * LD + qq], apq = A[pp * LD + qq];
                float c = 1.f, s = 0.f;
                const float thr = 1.1920928955078125e-07f * sqrtf(fabsf(app * aqq)) + abs_floor;
                if (fabsf(apq) > thr) {
                    const float theta = (aqq - app) / (2.f * apq);
                    // tan of the rotation angle, the root of t^2 + 2 theta t - 1 = 0 of
                    // smaller magnitude (1/(2 theta) once theta^2 would overflow)
                    const float t = fabsf(theta) > 1e18f
                                        ? 0.5f / theta
                                        : (theta >= 0.f ? 1.f : -1.f) /
                                              (fabsf(theta) + sqrtf(1.f + theta * theta));
                    c = 1.f / sqrtf(1.f + t * t);
                    s = t * c;
                    *flag = 1;
                }
                rp[tid] = pp;
                rq[tid] = qq;
                rc[tid] = c;
                rs[tid] = s;
            }
            __syncthreads();
            // columns: A <- A J, V <- V J
            for (int u = tid; u < D * H; u += kThreads) {
                const int m = u % H, r = u / H;
                const int pp = rp[m], qq = rq[m];
                const float c = rc[m], s = rs[m];
                const float x = A[r * LD + pp], y = A[r * LD + qq];
                A[r * LD + pp] = c * x - s * y;
                A[r * LD + qq] = s * x + c * y;
                const float vx = V[r * LD + pp], vy = V[r * LD + qq];
                V[r * LD + pp] = c * vx - s * vy;
                V[r * LD + qq] = s * vx + c * vy;
            }
            __syncthreads();
            // rows: A <- J^T A
            for (int u = tid; u < D * H; u += kThreads) {
                const int m = u % H, r = u / H;
                const int pp = rp[m], qq = rq[m];
                const float c = rc[m], s = rs[m];
                const float x = A[pp * LD + r], y = A[qq * LD + r];
                A[pp * LD + r] = c * x - s * y;
                A[qq * LD + r] = s * x + c * y;
            }
            __syncthreads();
        }
        if (*flag == 0) break;
        __syncthreads();
    }
    float *Vo = a.V + (int64_t)p * D * D;
    for (int e = tid; e < D * D; e += kThreads) Vo[e] = V[(e / D) * LD + e % D];
    if (tid < D) a.lam[(int64_t)p * D + tid] = A[tid * LD + tid];
}

// ------------------------------------------------ 4. pair loss and merge maps

struct LossArgs {
    const float *SG;     // [h_kt + P][D][D]
    const float *V;      // [P][D][D]
    const float *lam;    // [P][D]
    float *Sp;           // [P][D][D] scratch: S^+
    float *Pm;           // [P][2][D][D]: P_a = S_a S^+, P_b = S_b S^+
    double *w;           // [h_kt][h_kt] pair losses (output)
    int h_kt;
    uint8_t pa[kMaxPairs], pb[kMaxPairs];
};

// C tile (i0, j0) of X Y (or X Y^T) with MFMA 16x16x4, operands read from
// global memory (each block's matrices are a few tens of KB, L2/L1 resident).
template <int D, bool YT>
__device__ __forceinline__ f32x4v tile_mm(const float *X, const float *Y, int i0, int j0, int lane,
                                          const float *colscale = nullptr) {
    const int k = lane >> 4, i = lane & 15;
    f32x4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int k0 = 0; k0 < D; k0 += 4) {
        float xa = X[(i0 + i) * D + k0 + k];
        if (colscale) xa *= colscale[k0 + k];
        const float yb = YT ? Y[(j0 + i) * D + k0 + k] : Y[(k0 + k) * D + j0 + i];
        acc = mfma4(xa, yb, acc);
    }
    return acc;
}

template <int D>
__device__ __forceinline__ void tile_store(float *C, f32x4v v, int i0, int j0, int lane) {
#pragma unroll
    for (int r = 0; r < 4; ++r) C[(i0 + 4 * (lane >> 4) + r) * D + j0 + (lane & 15)] = v[r];
}

// One block per pair: S^+ from the eigenpairs (cutoff kEigRtol * max eigenvalue),
// P_a, P_b, and the pair's eq. 13 cost as <G P_b, P_b S_a> + <G P_a, P_a S_b>.
template <int D>
__global__ __launch_bounds__(kThreads) void k_pair_loss(LossArgs a) {
    constexpr int NB = D / 16;
    __shared__ float inv[D];
    __shared__ double dsum[4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int p = blockIdx.x;
    const int ia = a.pa[p], ib = a.pb[p];
    const int P = a.h_kt * (a.h_kt - 1) / 2;
    const float *Sa = a.SG + (int64_t)ia * D * D;
    const float *Sb = a.SG + (int64_t)ib * D * D;
    const float *G = a.SG + (int64_t)(a.h_kt + p) * D * D;
    const float *V = a.V + (int64_t)p * D * D;
    const float *lam = a.lam + (int64_t)p * D;
    float *Sp = a.Sp + (int64_t)p * D * D;
    float *Pa = a.Pm + (int64_t)p * 2 * D * D;
    float *Pb = Pa + D * D;

    if (tid < 64) {
        float m = -INFINITY;
        for (int e = tid; e < D; e += 64) m = fmaxf(m, lam[e]);
        m = wave_max(m);
        for (int e = tid; e < D; e += 64) {
            const float l = lam[e];
            inv[e] = (m > 0.f && l > kEigRtol * m) ? 1.f / l : 0.f;
        }
    }
    __syncthreads();
    // S^+ = V diag(inv) V^T
    for (int t = wave; t < NB * NB; t += 4) {
        const int i0 = (t / NB) * 16, j0 = (t % NB) * 16;
        tile_store<D>(Sp, tile_mm<D, true>(V, V, i0, j0, lane, inv), i0, j0, lane);
    }
    __syncthreads();
    for (int t = wave; t < 2 * NB * NB; t += 4) {
        const int which = t / (NB * NB), tt = t % (NB * NB);
        const int i0 = (tt / NB) * 16, j0 = (tt % NB) * 16;
        tile_store<D>(which ? Pb : Pa, tile_mm<D, false>(which ? Sb : Sa, Sp, i0, j0, lane), i0, j0,
                      lane);
    }
    __syncthreads();
    double part = 0.0;
    for (int t = wave; t < 2 * NB * NB; t += 4) {
        const int which = t / (NB * NB), tt = t % (NB * NB);
        const int i0 = (tt / NB) * 16, j0 = (tt % NB) * 16;
        const float *Pm = which ? Pa : Pb;           // term a uses P_b, term b uses P_a
        const float *Sx = which ? Sb : Sa;
        const f32x4v u = tile_mm<D, false>(G, Pm, i0, j0, lane);
        const f32x4v v = tile_mm<D, false>(Pm, Sx, i0, j0, lane);
#pragma unroll
        for (int r = 0; r < 4; ++r) part += (double)u[r] * (double)v[r];
    }
    for (int o = 32; o > 0; o >>= 1) part += __shfl_xor(part, o);
    if (lane == 0) dsum[wave] = part;
    __syncthreads();
    if (tid == 0) {
        const double L = dsum[0] + dsum[1] + dsum[2] + dsum[3];
        a.w[ia * a.h_kt + ib] = L;
        a.w[ib * a.h_kt + ia] = L;
    }
    if (p == 0 && tid < a.h_kt) a.w[tid * a.h_kt + tid] = 0.0;
    (void)P;
}

// ------------------------------------------------------------ 5. matching

struct MatchArgs {
    const double *w;     // [h_kt][h_kt]
    double *dp;          // [2^h_kt]
    uint8_t *choice;     // [2^h_kt]
    int32_t *pairs;      // [h_kt/2][2] output
    double *total;       // [1] output
    int h_kt;
    int forced;          // 1: take pairs from fa/fb instead of optimising
    uint8_t fa[kMaxHeads / 2], fb[kMaxHeads / 2];
};

// Minimum-weight perfect matching by dynamic programming over head subsets:
// best(M) = min over j in M, j != i (i = lowest head of M) of w(i, j) + best(M \ {i, j}),
// evaluated level by level (|M| = 2, 4, ...).  Ties go to the smallest j.
__global__ __launch_bounds__(kThreads) void k_match(MatchArgs a) {
    const int tid = threadIdx.x;
    const int h = a.h_kt;
    if (a.forced) {
        if (tid == 0) {
            double tot = 0.0;
            for (int i = 0; i < h / 2; ++i) {
                a.pairs[2 * i] = a.fa[i];
                a.pairs[2 * i + 1] = a.fb[i];
                tot += a.w[a.fa[i] * h + a.fb[i]];
            }
            *a.total = tot;
        }
        return;
    }
    const uint32_t full = (1u << h) - 1u;
    if (tid == 0) a.dp[0] = 0.0;
    __syncthreads();
    for (int lev = 2; lev <= h; lev += 2) {
        for (uint32_t m = tid; m <= full; m += kThreads) {
            if (__popc(m) != lev) continue;
            const int i = __ffs(m) - 1;
            double best = INFINITY;
            int bj = 0;
            for (int j = i + 1; j < h; ++j) {
                if (!((m >> j) & 1u)) continue;
                const double c = a.w[i * h + j] + a.dp[m ^ (1u << i) ^ (1u << j)];
                if (c < best) { best = c; bj = j; }
            }
            a.dp[m] = best;
            a.choice[m] = (uint8_t)bj;
        }
        __syncthreads();
    }
    if (tid == 0) {
        uint32_t m = full;
        int k = 0;
        while (m && k < h / 2) {                   // bounded even if a cost was NaN
            const int i = __ffs(m) - 1;
            const int j = a.choice[m];
            a.pairs[2 * k] = i;
            a.pairs[2 * k + 1] = j;
            ++k;
            m ^= (1u << i) | (1u << j);
        }
        *a.total = a.dp[full];
    }
}

// ------------------------------------------------------- 6. merged weights

struct WeightArgs {
    const uint16_t *W;   // [h_kt*D][dm] bf16 teacher key projection
    const float *Pm;     // [P][2][D][D]
    const int32_t *pairs;  // [h_kt/2][2]
    float *out;          // [h_kt/2*D][dm] fp32 merged projection
    int dm, h_kt;
};

// out row i*D + c, column x = sum_e W[a*D+e][x] P_a[e][c] + W[b*D+e][x] P_b[e][c]
// (eq. 15 in the weight layout: merged head i = pair (a, b) = pairs[i]).
template <int D>
__global__ __launch_bounds__(kThreads) void k_merged_weight(WeightArgs a) {
    extern __shared__ float sm[];
    float *Pa = sm, *Pb = sm + D * D;
    const int tid = threadIdx.x;
    const int hi = blockIdx.x;
    const int ia = a.pairs[2 * hi], ib = a.pairs[2 * hi + 1];
    if (ia < 0 || ib <= ia || ib >= a.h_kt) return;      // uniform per block
    const int p = ia * (2 * a.h_kt - ia - 1) / 2 + (ib - ia - 1);
    const float *src = a.Pm + (int64_t)p * 2 * D * D;
    for (int e = tid; e < 2 * D * D; e += kThreads) sm[e] = src[e];
    __syncthreads();
    const int x = blockIdx.y * kThreads + tid;
    if (x >= a.dm) return;
    float acc[D];
#pragma unroll
    for (int c = 0; c < D; ++c) acc[c] = 0.f;
    for (int e = 0; e < D; ++e) {
        const float wa = __uint_as_float((uint32_t)a.W[(int64_t)(ia * D + e) * a.dm + x] << 16);
        const float wb = __uint_as_float((uint32_t)a.W[(int64_t)(ib * D + e) * a.dm + x] << 16);
#pragma unroll
        for (int c = 0; c < D; ++c) acc[c] += wa * Pa[e * D + c] + wb * Pb[e * D + c];
    }
    float *o = a.out + (int64_t)hi * D * a.dm + x;
#pragma unroll
    for (int c = 0; c < D; ++c) o[(int64_t)c * a.dm] = acc[c];
}

}  // namespace merge
}  // namespace saga
