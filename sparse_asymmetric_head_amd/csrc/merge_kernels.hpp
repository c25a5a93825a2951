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
//      and G for every head pair                  (bf16 MFMA: exact products for
//      the queries, a split high/low bf16 pair for the fp32 key differences),
// and the rest is small dense algebra per head pair (a rank-revealing Cholesky
// for the pseudoinverse, a handful of d x d products) plus a 2^h_kt-state
// matching.
#pragma once

#include "saga_device.hpp"

namespace saga {
namespace merge {

constexpr int kThreads = 256;
constexpr int kMaxHeads = 16;                       // teacher key heads (h_kt)
constexpr int kMaxPairs = kMaxHeads * (kMaxHeads - 1) / 2;
constexpr float kPivotRtol = 6.103515625e-05f;      // 2^-14: rank cut, relative to max_i S_ii

typedef float f32x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4v mfma4(float a, float b, f32x4v c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// ------------------------------------------------------------------ 1. keys

struct ProjArgs {
    const uint16_t *X;  // [n][dm] bf16
    const uint16_t *W;  // [cols][dm] bf16 (row r*D + c = channel c of teacher key head r)
    float *Kt;          // fp32 keys in key-fragment order (kfrag_index); tokens n .. ldt-1 written as zero
    int64_t n, ldt;     // ldt: n rounded up to 128
    int dm;
    int cols;
};

constexpr int kPBM = 128, kPBN = 128, kPBK = 64;    // token padding, block columns, k-stage

// Key-fragment order of the projected keys: channel c (of all h_kt d) and token t
// (of ldt) sit in the 2 KB block of 16-channel group c / 16 and 32-token group
// t / 32; inside it, lane l = 16 q + i (channel 16 (c / 16) + i, tokens 8 q ..
// 8 q + 7 of the group) finds its first four tokens at 16-byte slot l and the
// next four at slot 64 + l.  A wave then reads an MFMA operand (16 channels x 32
// tokens, as the key-difference Gram needs it) as two contiguous 1 KB loads, and
// the projection's four-token stores of 16 consecutive channels are contiguous.
__host__ __device__ __forceinline__ int64_t kfrag_index(int64_t c, int64_t t, int64_t ldt) {
    const int64_t blk = (c >> 4) * (ldt >> 5) + (t >> 5);
    const int tt = (int)(t & 31);
    return blk * 512 + ((tt >> 2) & 1) * 256 + (16 * (tt >> 3) + (int)(c & 15)) * 4 + (tt & 3);
}

// LDS tile [rows][64 k] bf16: row = 8 chunks of 16 B, chunk c of row r stored
// at chunk position c ^ (r & 7), so the 16 rows one MFMA operand read touches
// fall on different banks.
__device__ __forceinline__ int swz(int row, int chunk) { return row * 8 + (chunk ^ (row & 7)); }

// Stages of the projection's LDS ring: 144 KB (BM = 256) or 128 KB (BM = 128).
__host__ __device__ constexpr int proj_stages(int bm) { return bm == 256 ? 3 : 4; }
__host__ __device__ constexpr int proj_threads(int bm) { return bm / 64 * 2 * 64; }
__host__ __device__ constexpr size_t proj_lds_bytes(int bm) {
    return (size_t)proj_stages(bm) * (bm + kPBN) * 8 * 16;
}

// s_waitcnt vmcnt(N) (the other counters left alone), N < 64.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier that leaves the vector-memory counter alone (__syncthreads
// waits for every outstanding load, the direct LDS loads of later stages too):
// the caller has waited for what it needs; LDS operations are complete first
// (lgkmcnt(0)), and the compiler keeps memory accesses on their side.
__device__ __forceinline__ void barrier_keep_loads() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// K = X W^T.  Block tile BM tokens x 128 columns, BM/64 x 2 waves of 64 x 64
// (4 x 4 MFMA 16x16x32 tiles each).  The X and W tiles of each 64-wide k-stage
// go through a ring of proj_stages(BM) LDS stages filled by direct global->LDS
// loads, so two (BM 256) or three (BM 128) stages are in flight while one is
// multiplied, with no staging registers and one barrier per stage.  Lane l of a
// direct load lands in LDS slot l of the load's 64 slots, so the XOR swizzle of
// the 16-byte chunks (swz) is made by the choice of each lane's source address.
template <int BM>
__global__ __launch_bounds__(proj_threads(BM)) void k_kproj(ProjArgs a) {
    constexpr int NW = proj_threads(BM) / 64;      // waves
    constexpr int S = proj_stages(BM);             // ring stages
    constexpr int SLOTS = (BM + kPBN) * 8;         // 16-byte chunks per stage
    constexpr int LPW = SLOTS / (64 * NW);         // direct loads per wave and stage
    static_assert(LPW * 64 * NW == SLOTS && (BM * 8) % 64 == 0, "stage split");
    extern __shared__ u32x4 ring[];                // [S][SLOTS]: X rows, then W rows
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t t0 = (int64_t)blockIdx.x * BM;
    const int n0 = blockIdx.y * kPBN;
    const int64_t last = a.n - 1;
    const int nk = a.dm / kPBK;

    // source of this lane's chunk in each of the wave's loads; rows past n read
    // the last token (their outputs are not kept)
    const uint16_t *src[LPW];
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
        const int sl = (wave * LPW + j) * 64 + lane;   // X or W for the whole wave: uniform
        if (sl < BM * 8) {
            const int row = sl >> 3, ch = (sl & 7) ^ (row & 7);
            int64_t t = t0 + row;
            t = t < last ? t : last;
            src[j] = a.X + t * a.dm + ch * 8;
        } else {
            const int row = (sl - BM * 8) >> 3, ch = (sl & 7) ^ (row & 7);
            src[j] = a.W + (int64_t)(n0 + row) * a.dm + ch * 8;
        }
    }
    auto issue = [&](int kt) {
        u32x4 *dst = ring + (kt % S) * SLOTS + wave * LPW * 64;
#pragma unroll
        for (int j = 0; j < LPW; ++j)
            __builtin_amdgcn_global_load_lds((const void *)(src[j] + kt * kPBK),
                                             (__attribute__((address_space(3))) void *)(dst + j * 64),
                                             16, 0, 0);
    };
    f32x4v acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4v{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int st = 0; st < S - 1; ++st)
        if (st < nk) issue(st);
    for (int kt = 0; kt < nk; ++kt) {
        // this wave's loads of stage kt are done once at most the later stages'
        // loads are outstanding; the barrier then makes every wave's part visible
        // and frees the slot of stage kt - 1 for stage kt + S - 1
        const int later = min(S - 2, nk - 1 - kt);
        if (later >= 2) wait_vmcnt<2 * LPW>();
        else if (later == 1) wait_vmcnt<LPW>();
        else wait_vmcnt<0>();
        barrier_keep_loads();
        if (kt + S - 1 < nk) issue(kt + S - 1);
        const u32x4 *As = ring + (kt % S) * SLOTS;
        const u32x4 *Bs = As + BM * 8;
#pragma unroll
        for (int s = 0; s < 2; ++s) {               // two k-steps of 32 per stage
            const int ch = s * 4 + (lane >> 4);
            bf16x8 af[4], bfr[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                af[i] = as_bf16x8(As[swz(wm * 64 + i * 16 + (lane & 15), ch)]);
                bfr[i] = as_bf16x8(Bs[swz(wn * 64 + i * 16 + (lane & 15), ch)]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j],
                                                                        0, 0, 0);
        }
    }
    // lane holds rows (tokens) 4*(lane/16)+r, column lane%16 of each 16 x 16 tile:
    // four consecutive tokens of one channel, one 16-byte store (zero past n,
    // nothing past the padded token count ldt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t t = t0 + wm * 64 + i * 16 + (lane >> 4) * 4;
        if (t >= a.ldt) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const f32x4v v = acc[i][j];
            const float4 o = {t + 0 < a.n ? v[0] : 0.f, t + 1 < a.n ? v[1] : 0.f,
                              t + 2 < a.n ? v[2] : 0.f, t + 3 < a.n ? v[3] : 0.f};
            *(float4 *)(a.Kt + kfrag_index(n0 + wn * 64 + j * 16 + (lane & 15), t, a.ldt)) = o;
        }
    }
}

// ------------------------------------------------------------ 2. Grams

struct GramArgs {
    const uint16_t *Q;   // [n][h_q][D] bf16 calibration queries
    const float *Kt;     // fp32 projected keys in key-fragment order (kfrag_index), zero past n
    int64_t ldt;         // a multiple of 128, >= n
    float *part;         // per-block partial sums: [item][chunk][D][D] of this launch's items
    int64_t n;
    int64_t chunk_tokens;
    int n_chunk;
    int h_q, h_kt;
    uint8_t pa[kMaxPairs], pb[kMaxPairs];  // pair p = (pa[p], pb[p]), pa < pb
};

// Tile groups of a Gram block: the (D/16)(D/16+1)/2 tiles I <= J of one item's
// second moment are dealt round-robin to gram_groups blocks (blockIdx.z) that
// read the same samples.  A query block holds all of them (d = 128: 144
// accumulator registers of the 512 a lane has at one wave per SIMD); a d = 128
// key-difference block holds a quarter, since its double-buffered fp32 loads
// and bf16 splits take most of the rest (measured: a half is slower).
__host__ __device__ constexpr int gram_groups(int D, bool is_q) {
    return D >= 128 ? (is_q ? 1 : 4) : 1;
}

constexpr int kGramStep = 32;   // samples per MFMA 16x16x32 k-step
constexpr int kGramWaves = kThreads / 64;
constexpr int kQtStride = 40;   // LDS row stride of the transposed query tile, bf16 (80 bytes)

// Round x to bf16 (nearest even) as the high part and the rounded remainder as
// the low part: x = hi + lo to about 2^-17 relative.
__device__ __forceinline__ void split_bf16(float x, __bf16 &hi, __bf16 &lo) {
    hi = (__bf16)x;
    lo = (__bf16)(x - (float)hi);
}

// One block per (item, token chunk, tile group).  MFMA 16x16x32 bf16 with the
// sample as the contraction index: lane (q = lane/16, i = lane%16) supplies, for
// feature block I, channel 16 I + i of samples 8 q .. 8 q + 7 as both the A
// (row) and the B (column) operand, so each instruction adds 32 samples' outer
// products to a 16 x 16 tile; only tiles I <= J are formed.
//  IS_Q: item r = blockIdx.y, S_r over the (token, query head of group r)
//   samples.  Query rows are channel-contiguous, so each wave stages 32 samples
//   through a wave-private LDS tile (lane (sg, c8) loads channels 8 c8 .. +7 of
//   samples 4 sg .. +3 and writes them as 4-sample runs of each channel; the
//   80-byte rows make the 16-byte fragment reads conflict-free).  bf16 inputs:
//   the products are exact.
//  else: item p = blockIdx.y, G_p over tokens of the fp32 key difference
//   K_a - K_b, read in key-fragment order (a lane's 8 tokens arrive in two
//   16-byte slots of contiguous 1 KB wave loads, no staging), split into bf16
//   high and low parts; hi hi + hi lo + lo hi per tile.
// Loads of the next step are issued before the current step's multiplies.  The
// block writes its tiles (and their mirror images) into the (item, chunk) partial.
template <int D, bool IS_Q>
__global__ __launch_bounds__(kThreads) void k_gram(GramArgs a) {
    constexpr int NB = D / 16;                     // feature blocks
    constexpr int NT = NB * (NB + 1) / 2;          // tiles I <= J
    constexpr int TG = gram_groups(D, IS_Q);
    constexpr int NA = (NT + TG - 1) / TG;         // accumulator tiles per block
    constexpr int NH = D / 64;                     // 8-channel chunks per lane (queries)
    __shared__ float red[NA * 256];
    __shared__ uint16_t qt[IS_Q ? kGramWaves : 1][IS_Q ? D * kQtStride : 1];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int q4 = lane >> 4, i16 = lane & 15;
    const int item = blockIdx.y;
    const int grp = blockIdx.z;
    const int64_t t_beg = (int64_t)blockIdx.x * a.chunk_tokens;

    f32x4v acc[NA];
#pragma unroll
    for (int t = 0; t < NA; ++t) acc[t] = f32x4v{0.f, 0.f, 0.f, 0.f};
    // tile t (row-major over I <= J) belongs to group t % TG, slot t / TG
    auto tiles = [&](auto &&fn) {
#pragma unroll
        for (int I = 0; I < NB; ++I)
#pragma unroll
            for (int J = I; J < NB; ++J) {
                const int t = I * NB - I * (I - 1) / 2 + (J - I);
                if (t % TG == grp) fn(I, J, t / TG);
            }
    };

    if constexpr (IS_Q) {
        const int lo = (item * a.h_q + a.h_kt - 1) / a.h_kt;     // first j with j*h_kt/h_q >= item
        const int g = ((item + 1) * a.h_q + a.h_kt - 1) / a.h_kt - lo;
        int64_t t_end = t_beg + a.chunk_tokens;
        t_end = t_end < a.n ? t_end : a.n;
        const int ntok = (int)(t_end > t_beg ? t_end - t_beg : 0);
        const int n_samp = ntok * g;
        const int per_wave = (n_samp + kGramWaves * kGramStep - 1) / (kGramWaves * kGramStep) * kGramStep;
        const int s_beg = wave * per_wave;
        const int s_end = min(s_beg + per_wave, n_samp);
        const int sg = lane >> 3, c8 = lane & 7;
        uint16_t *tile = qt[wave];
        // raw[h][u]: channels 8 (c8 + 8 h) .. +7 of sample s0 + 4 sg + u
        auto load = [&](int s0, u32x4 (&raw)[NH][4]) {
            int s = s0 + 4 * sg;
            int tl = s / g, jj = s - tl * g;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const bool ok = s + u < s_end;
                const uint16_t *src = a.Q + ((t_beg + (ok ? tl : 0)) * a.h_q + lo + (ok ? jj : 0)) * D + 8 * c8;
#pragma unroll
                for (int h = 0; h < NH; ++h) {
                    const u32x4 v = ld16(src + 64 * h);
                    raw[h][u] = ok ? v : u32x4{0u, 0u, 0u, 0u};
                }
                if (++jj == g) { jj = 0; ++tl; }
            }
        };
        auto process = [&](const u32x4 (&raw)[NH][4]) {
#pragma unroll
            for (int h = 0; h < NH; ++h)
#pragma unroll
                for (int w2 = 0; w2 < 4; ++w2) {          // channels 2 w2, 2 w2 + 1 of the chunk
                    const uint32_t x0 = raw[h][0][w2], x1 = raw[h][1][w2];
                    const uint32_t x2 = raw[h][2][w2], x3 = raw[h][3][w2];
                    const uint2 ev = {(x0 & 0xffffu) | (x1 << 16), (x2 & 0xffffu) | (x3 << 16)};
                    const uint2 od = {(x0 >> 16) | (x1 & 0xffff0000u), (x2 >> 16) | (x3 & 0xffff0000u)};
                    const int ch = 8 * (c8 + 8 * h) + 2 * w2;
                    *(uint2 *)(tile + ch * kQtStride + 4 * sg) = ev;
                    *(uint2 *)(tile + (ch + 1) * kQtStride + 4 * sg) = od;
                }
            bf16x8 f[NB];
#pragma unroll
            for (int I = 0; I < NB; ++I)
                f[I] = as_bf16x8(*(const u32x4 *)(tile + (16 * I + i16) * kQtStride + 8 * q4));
            tiles([&](int I, int J, int sl) {
                acc[sl] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f[I], f[J], acc[sl], 0, 0, 0);
            });
        };
        if (s_beg < s_end) {
            u32x4 ra[NH][4], rb[NH][4];
            load(s_beg, ra);
            for (int s0 = s_beg;; s0 += 2 * kGramStep) {
                load(s0 + kGramStep, rb);
                process(ra);
                if (s0 + kGramStep >= s_end) break;
                load(s0 + 2 * kGramStep, ra);
                process(rb);
                if (s0 + 2 * kGramStep >= s_end) break;
            }
        }
    } else {
        const int ka = a.pa[item], kb = a.pb[item];
        int64_t t_end = t_beg + a.chunk_tokens;
        t_end = t_end < a.ldt ? t_end : a.ldt;                  // past n the keys are zero
        const int64_t ntok = t_end > t_beg ? t_end - t_beg : 0;  // a multiple of 128
        const int64_t per_wave = ntok / kGramWaves;
        const int64_t w_beg = t_beg + wave * per_wave, w_end = w_beg + per_wave;
        // raw[I][0..1]: tokens t0 + 8 q4 .. +7 of channel 16 I + i16, heads a, b:
        // 16-byte slots lane and 64 + lane of the (channel group, token group)
        // block, so each load of the wave is 1 KB contiguous
        const int64_t gstride = (a.ldt >> 5) * 512;   // floats per 16-channel group
        const float *Ka = a.Kt + (int64_t)(ka * D / 16) * gstride + lane * 4;
        const float *Kb = a.Kt + (int64_t)(kb * D / 16) * gstride + lane * 4;
        auto load = [&](int64_t t0, float4 (&ra)[NB][2], float4 (&rb)[NB][2]) {
#pragma unroll
            for (int I = 0; I < NB; ++I) {
                const int64_t off = I * gstride + (t0 >> 5) * 512;
                ra[I][0] = *(const float4 *)(Ka + off);
                ra[I][1] = *(const float4 *)(Ka + off + 256);
                rb[I][0] = *(const float4 *)(Kb + off);
                rb[I][1] = *(const float4 *)(Kb + off + 256);
            }
        };
        auto process = [&](const float4 (&ra)[NB][2], const float4 (&rb)[NB][2]) {
            bf16x8 hi[NB], lo[NB];
#pragma unroll
            for (int I = 0; I < NB; ++I) {
                const float x[8] = {ra[I][0].x - rb[I][0].x, ra[I][0].y - rb[I][0].y,
                                    ra[I][0].z - rb[I][0].z, ra[I][0].w - rb[I][0].w,
                                    ra[I][1].x - rb[I][1].x, ra[I][1].y - rb[I][1].y,
                                    ra[I][1].z - rb[I][1].z, ra[I][1].w - rb[I][1].w};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    __bf16 h, l;
                    split_bf16(x[e], h, l);
                    hi[I][e] = h;
                    lo[I][e] = l;
                }
            }
            tiles([&](int I, int J, int sl) {
                acc[sl] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi[I], hi[J], acc[sl], 0, 0, 0);
                acc[sl] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi[I], lo[J], acc[sl], 0, 0, 0);
                acc[sl] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo[I], hi[J], acc[sl], 0, 0, 0);
            });
        };
        if (w_beg < w_end) {
            float4 aa[NB][2], ab[NB][2], ba[NB][2], bb[NB][2];
            load(w_beg, aa, ab);
            for (int64_t t0 = w_beg;; t0 += 2 * kGramStep) {
                if (t0 + kGramStep < w_end) load(t0 + kGramStep, ba, bb);
                process(aa, ab);
                if (t0 + kGramStep >= w_end) break;
                if (t0 + 2 * kGramStep < w_end) load(t0 + 2 * kGramStep, aa, ab);
                process(ba, bb);
                if (t0 + 2 * kGramStep >= w_end) break;
            }
        }
    }

    // Sum the four waves' tiles in LDS (slot-major, 256 words per tile), one wave
    // at a time; lane holds rows 4 q4 + r, column i16 of each tile.
    for (int w = 0; w < kGramWaves; ++w) {
        if (wave == w) {
#pragma unroll
            for (int q = 0; q < NA; ++q)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int e = q * 256 + (4 * q4 + r) * 16 + i16;
                    red[e] = (w == 0 ? 0.f : red[e]) + acc[q][r];
                }
        }
        __syncthreads();
    }
    // write the block's tiles and their mirror images into the partial
    float *dst = a.part + ((int64_t)item * a.n_chunk + blockIdx.x) * (D * D);
    const int rr = tid >> 4, cc = tid & 15;              // 256 threads: one entry each
    tiles([&](int I, int J, int sl) {
        const float v = red[sl * 256 + rr * 16 + cc];
        const int row = 16 * I + rr, col = 16 * J + cc;
        dst[row * D + col] = v;
        if (I != J) dst[col * D + row] = v;
    });
}

struct ReduceArgs {
    const float *part;   // [h_kt][nq][D*D] then [P][nd][D*D]
    float *out;          // [h_kt + P][D*D]
    int h_kt, nq, nd;
    int dd;              // D*D
};

// Fixed-order fp64 sum of the per-block partials (deterministic).
__global__ __launch_bounds__(kThreads) void k_gram_reduce(ReduceArgs a) {
    const int e = blockIdx.x * kThreads + threadIdx.x;
    if (e >= a.dd) return;
    const int item = blockIdx.y;
    const bool q = item < a.h_kt;
    const int nc = q ? a.nq : a.nd;
    const int64_t base = q ? (int64_t)item * a.nq * a.dd
                           : ((int64_t)a.h_kt * a.nq + (int64_t)(item - a.h_kt) * a.nd) * a.dd;
    const float *p = a.part + base + e;
    double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
    int c = 0;
#pragma unroll 4                       // 16 loads in flight
    for (; c + 4 <= nc; c += 4) {
        s0 += (double)p[(int64_t)(c + 0) * a.dd];
        s1 += (double)p[(int64_t)(c + 1) * a.dd];
        s2 += (double)p[(int64_t)(c + 2) * a.dd];
        s3 += (double)p[(int64_t)(c + 3) * a.dd];
    }
    for (; c < nc; ++c) s0 += (double)p[(int64_t)c * a.dd];
    a.out[(int64_t)item * a.dd + e] = (float)((s0 + s1) + (s2 + s3));
}

// --------------------------------------------- 3. pseudoinverse per pair

struct PinvArgs {
    const float *SG;     // [h_kt + P][D][D]: S_r, then G_p
    float *Sp;           // [P][D][D] output: (S_a + S_b)^+
    int *rank;           // [P] numerical rank
    int h_kt;
    uint8_t pa[kMaxPairs], pb[kMaxPairs];
};

// Threads of a pseudoinverse block: each thread of the pivoted path holds 16
// entries (one register vector) of the D x D working matrix, so a step's update
// is short and the block's waves split it evenly (d = 64: 256 threads, d = 128:
// 1024); the blocked path uses the same count.
__host__ __device__ constexpr int pinv_threads(int D) { return D * D / 16; }

// ---- fast path: S^-1 for a comfortably full-rank S by blocked sweeps
//
// The symmetric sweep of a block b of rows/columns (the SWEEP operator on a
// block) maps, with B = A_bb^-1,
//     A_ij -> A_ij - A_ib B A_bj   (i, j outside b),
//     A_bj -> B A_bj,  A_ib -> A_ib B,  A_bb -> -B,
// and sweeping every block in turn leaves -A^-1 (the pivoted path below sweeps
// one row at a time in pivot order).  Here a block is one 16 x 16 tile, in
// natural order, without pivoting.  The matrix stays in registers as 16 x 16
// tiles in the MFMA output layout; one wave inverts each diagonal tile by 16
// scalar sweeps with cross-lane moves only (no LDS, no barrier), the panel
// product B A_bj and the rank-16 update run on fp32 MFMA, and the update of
// the next tile row goes first, so the next diagonal inversion overlaps the
// rest of the update (three barriers per block).
// The result is used only when the pivoted rule would also find full rank:
// the largest diagonal of every Schur complement of S is at least
// lambda_min(S) >= 1 / trace(S^-1), so if 1 / trace(S^-1) clears the rank cut
// (kPivotRtol * max_i S_ii) by kFastMargin, S^+ = S^-1.  Otherwise (or on a
// non-positive tile pivot) the block starts over on the pivoted path.
constexpr float kFastMargin = 4.0f;

typedef unsigned int u32x2v __attribute__((ext_vector_type(2)));

// x of lane K of each 16-lane row, to every lane of that row (DPP row_newbcast)
template <int K>
__device__ __forceinline__ float row_newbcast(float x) {
    return __int_as_float(
        __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x150 + K, 0xF, 0xF, false));
}

// x of 16-lane row G, to the same lane of all four rows: the row-pair swap gives
// rows (0, 0, 2, 2) and (1, 1, 3, 3), the half swap of one of those gives
// (y0, y1, y0, y1) and (y2, y3, y2, y3)
template <int G>
__device__ __forceinline__ float rows_bcast(float x) {
    const unsigned u = __float_as_uint(x);
    const u32x2v h = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const unsigned y = (G & 1) ? h[1] : h[0];
    const u32x2v f = __builtin_amdgcn_permlane32_swap(y, y, false, false);
    return __uint_as_float((G & 2) ? f[1] : f[0]);
}

// A symmetric 16 x 16 tile in one wave: lane l holds row r = l % 16, columns
// 4 cq .. 4 cq + 3 with cq = l / 16, in w[0..3].  One sweep on pivot K: row K
// for the lane's own columns comes from lane K of its 16-lane row, column K at
// row r from 16-lane row K / 4 (same lane position), the pivot by readlane.
template <int K>
__device__ __forceinline__ void tile_sweep(float (&w)[4], int r, int cq, bool &ok) {
    constexpr int KQ = K >> 2, KV = K & 3;
    const float pk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w[KV]), K + 16 * KQ));
    float rk[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) rk[v] = row_newbcast<K>(w[v]);  // A(K, 4 cq + v)
    const float cr = rows_bcast<KQ>(w[KV]);                      // A(r, K)
    ok = ok && pk > 0.f && pk < INFINITY;                        // wave-uniform
    const float ip = __builtin_amdgcn_rcpf(pk);                 // 1 ulp
    const bool rowk = r == K;
    const float g = rowk ? 0.f : cr * ip;
    const float sc = rowk ? ip : 1.f;
#pragma unroll
    for (int v = 0; v < 4; ++v) w[v] = fmaf(-g, rk[v], w[v] * sc);
    const float colk = rowk ? -ip : cr * ip;
    w[KV] = (cq == KQ) ? colk : w[KV];
}
template <int K>
struct TileSweeps {
    static __device__ __forceinline__ void run(float (&w)[4], int r, int cq, bool &ok) {
        tile_sweep<K>(w, r, cq, ok);
        TileSweeps<K + 1>::run(w, r, cq, ok);
    }
};
template <>
struct TileSweeps<16> {
    static __device__ __forceinline__ void run(float (&)[4], int, int, bool &) {}
};

// LDS floats of the blocked path: two tile rows, two panel products, two B,
// a private 16 x 16 tile per wave, S_a + S_b
__host__ __device__ constexpr int blocked_lds_floats(int D) {
    return 4 * 16 * (D + 16) + 2 * 16 * 20 + (D * D / 16 / 64) * 256 + D * (D + 4);
}

// S^-1 of pair p by blocked sweeps; true (block-uniform) when it is S^+ and has
// been written, false when the pair needs the pivoted path.
template <int D>
__device__ __forceinline__ bool pair_inv_blocked(const PinvArgs &a, int p, float *sm) {
    constexpr int TH = pinv_threads(D);
    constexpr int NW = TH / 64;          // waves (4 or 16); wave 0 only inverts diagonal tiles
    constexpr int NTW = NW - 1;          // waves holding tiles
    constexpr int NB = D / 16;           // tiles per row
    constexpr int NT = (NB * NB + NTW - 1) / NTW;  // tile slots per wave (6 or 5)
    constexpr int LP = D + 16;           // row stride of a tile row: 16 x 4 MFMA reads hit 64 banks
    constexpr int LB = 20;               // row stride of B
    float *const pan = sm;               // [2][16][LP] tile row b before the sweep of block b
    float *const pmb = sm + 2 * 16 * LP; // [2][16][LP] B times that row
    float *const bmb = sm + 4 * 16 * LP; // [2][16][LB] B = (diagonal tile)^-1
    float *const own = bmb + 2 * 16 * LB;  // [NW][16][16] a wave's private copy of one B A_bj
    constexpr int LL = D + 4;
    float *const ls = own + NW * 256;    // [D][LL] S_a + S_b
    __shared__ float red[NW], redm[NW];
    __shared__ int bad;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar: tile indices, LDS slots
    const int li = lane & 15, lk = lane >> 4;  // MFMA operand / output lane roles
    const float *Sa = a.SG + (int64_t)a.pa[p] * D * D;
    const float *Sb = a.SG + (int64_t)a.pb[p] * D * D;
    // slot q of wave w >= 1 holds tile t = (w - 1) + NTW q (if t < NB^2), tile
    // (t / NB, t % NB); lane holds rows 4 lk + u of column li of it (the MFMA
    // output layout)
    auto tile_of = [&](int q) { return wave == 0 ? NB * NB : (wave - 1) + NTW * q; };
    // S_a + S_b through LDS (coalesced 16-byte loads), then the symmetric part
    // of the wave's tiles
#pragma unroll
    for (int i = 0; i < D * D / 4 / TH; ++i) {
        const int e = 4 * (tid + TH * i), r = e / D, c = e % D;
        const float4 x = *(const float4 *)(Sa + e), y = *(const float4 *)(Sb + e);
        *(float4 *)(ls + r * LL + c) = make_float4(x.x + y.x, x.y + y.y, x.z + y.z, x.w + y.w);
    }
    __syncthreads();
    f32x4v C[NT];
    float dmx = 0.f;
#pragma unroll
    for (int q = 0; q < NT; ++q) {
        const int t = tile_of(q);
        if (t >= NB * NB) continue;
        const int r0 = (t / NB) * 16, c0 = (t % NB) * 16;
        const float4 tt = *(const float4 *)(ls + (c0 + li) * LL + r0 + 4 * lk);  // S(c, r)
        const float tr4[4] = {tt.x, tt.y, tt.z, tt.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int r = r0 + 4 * lk + u, c = c0 + li;
            C[q][u] = 0.5f * (ls[r * LL + c] + tr4[u]);
            if (r == c) dmx = fmaxf(dmx, C[q][u]);
        }
    }
    auto publish = [&](int q, float *P) {
        const int tj = tile_of(q) % NB;
#pragma unroll
        for (int u = 0; u < 4; ++u) P[(4 * lk + u) * LP + tj * 16 + li] = C[q][u];
    };
    // B A_sj (16 x 16) from the tile row P and B
    auto panel_tile = [&](const float *P, const float *Bm, int j) {
        f32x4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k0 = 0; k0 < 16; k0 += 4)
            acc = mfma4(Bm[li * LB + k0 + lk], P[(k0 + lk) * LP + j * 16 + li], acc);
        return acc;
    };
    // the sweep of block s on the wave's tiles outside tile row `skip`
    auto sweep_block = [&](int s, int skip) {
        const float *P = pan + (s & 1) * 16 * LP;
        const float *M = pmb + (s & 1) * 16 * LP;
        const float *Bm = bmb + (s & 1) * 16 * LB;
#pragma unroll
        for (int q = 0; q < NT; ++q) {
            const int t = tile_of(q), ti = t / NB, tj = t % NB;
            if (t >= NB * NB || ti == skip) continue;
            const bool ib = ti == s, jb = tj == s;
            if (ib && jb) {
#pragma unroll
                for (int u = 0; u < 4; ++u) C[q][u] = -Bm[(4 * lk + u) * LB + li];
            } else if (ib) {
#pragma unroll
                for (int u = 0; u < 4; ++u) C[q][u] = M[(4 * lk + u) * LP + tj * 16 + li];
            } else if (jb) {           // A_is B = (B A_si)^T
                const float4 v = *(const float4 *)(M + li * LP + ti * 16 + 4 * lk);
                C[q][0] = v.x;
                C[q][1] = v.y;
                C[q][2] = v.z;
                C[q][3] = v.w;
            } else {                   // A_ij - A_is (B A_sj), A_is = A_si^T
                f32x4v acc = C[q];
#pragma unroll
                for (int k0 = 0; k0 < 16; k0 += 4)
                    acc = mfma4(-P[(k0 + lk) * LP + ti * 16 + li], M[(k0 + lk) * LP + tj * 16 + li], acc);
                C[q] = acc;
            }
        }
    };

    // (a DPP reduction: the lane-shuffle one keeps its lane addresses live
    // across the loop and spills them)
    dmx = fkey_inv(wave_max_u32_dpp(fkey(dmx)));
    if (lane == 0) redm[wave] = dmx;   // read at the end
    if (tid == 0) bad = 0;
#pragma unroll
    for (int q = 0; q < NT; ++q) {
        const int t = tile_of(q);
        if (t < NB) publish(q, pan);
    }
    __syncthreads();

#pragma unroll 1
    for (int b = 0; b < NB; ++b) {
        const float *P = pan + (b & 1) * 16 * LP;
        float *M = pmb + (b & 1) * 16 * LP;
        float *Bm = bmb + (b & 1) * 16 * LB;
        // 1. wave 0 inverts the diagonal tile; the others finish the sweep of
        //    block b - 1 on their tiles outside row b (row b went first)
        if (wave == 0) {
            const int r = lane & 15, cq = lane >> 4;
            const float4 x = *(const float4 *)(P + r * LP + b * 16 + 4 * cq);
            float w[4] = {x.x, x.y, x.z, x.w};
            bool ok = true;
            TileSweeps<0>::run(w, r, cq, ok);
            *(float4 *)(Bm + r * LB + 4 * cq) = make_float4(-w[0], -w[1], -w[2], -w[3]);
            if (!ok && lane == 0) bad = 1;
        } else if (b > 0) {
            sweep_block(b - 1, b);
        }
        __syncthreads();
        // 2. B A_bj for every j != b, and the sweep of block b on tile row b + 1,
        //    published for the next block.  The holder of tile (b+1, j) forms
        //    the B A_bj it needs itself (j = b+1 for j = b), writes it to the
        //    shared panel product (or, for j = b, to its private copy) and reads
        //    it back in the operand layout.
        if (b + 1 < NB) {
#pragma unroll
            for (int q = 0; q < NT; ++q) {
                const int t = tile_of(q), ti = t / NB, tj = t % NB;
                if (t >= NB * NB || ti != b + 1) continue;
                const int jp = tj == b ? b + 1 : tj;
                const f32x4v pm = panel_tile(P, Bm, jp);
                float *const dst = tj == b ? own + wave * 256 : M + jp * 16;
                const int ld = tj == b ? 16 : LP;
#pragma unroll
                for (int u = 0; u < 4; ++u) dst[(4 * lk + u) * ld + li] = pm[u];
                if (tj == b) {         // A_(b+1)b B = (B A_b(b+1))^T
                    const float4 v = *(const float4 *)(dst + li * ld + 4 * lk);
                    C[q][0] = v.x;
                    C[q][1] = v.y;
                    C[q][2] = v.z;
                    C[q][3] = v.w;
                } else {
                    f32x4v acc = C[q];
#pragma unroll
                    for (int k0 = 0; k0 < 16; k0 += 4)
                        acc = mfma4(-P[(k0 + lk) * LP + ti * 16 + li], dst[(k0 + lk) * ld + li], acc);
                    C[q] = acc;
                }
                publish(q, pan + ((b + 1) & 1) * 16 * LP);
            }
        } else {
            for (int j = wave; j < NB; j += NW) {
                if (j == b) continue;
                const f32x4v pm = panel_tile(P, Bm, j);
#pragma unroll
                for (int u = 0; u < 4; ++u) M[(4 * lk + u) * LP + j * 16 + li] = pm[u];
            }
        }
        __syncthreads();
    }
    sweep_block(NB - 1, NB);

    // C = -S^-1: trace(S^-1) = -sum of the diagonal
    float tr = 0.f;
#pragma unroll
    for (int q = 0; q < NT; ++q) {
        const int t = tile_of(q), ti = t / NB, tj = t % NB;
        if (t >= NB * NB) continue;
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (ti == tj && 4 * lk + u == li) tr -= C[q][u];
    }
    tr = wave_sum(tr);
    if (lane == 0) red[wave] = tr;
    __syncthreads();                   // also: every read of the LDS above is done
    tr = 0.f;
    dmx = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        tr += red[w];
        dmx = fmaxf(dmx, redm[w]);
    }
    const bool use = !bad && tr > 0.f && tr < INFINITY &&
                     1.f / tr >= kFastMargin * kPivotRtol * dmx;  // block-uniform
    if (!use) {
        if (tid == 0) a.rank[p] = 0;   // the pivoted kernel takes this pair
        return false;
    }
    float *out = a.Sp + (int64_t)p * D * D;
#pragma unroll
    for (int q = 0; q < NT; ++q) {
        const int t = tile_of(q), ti = t / NB, tj = t % NB;
        if (t >= NB * NB) continue;
#pragma unroll
        for (int u = 0; u < 4; ++u) out[(ti * 16 + 4 * lk + u) * D + tj * 16 + li] = -C[q][u];
    }
    if (tid == 0) a.rank[p] = D;
    return true;
}

// C tile (i0, j0) of a product of two LDS matrices (row stride LD), MFMA 16x16x4:
// C[i][j] = sum_k X(i, k) Y(k, j) with X(i, k) = XT ? X[k][i] : X[i][k] and
// Y(k, j) = YT ? Y[j][k] : Y[k][j].
template <int D, int LD, bool XT, bool YT>
__device__ __forceinline__ f32x4v lds_tile_mm(const float *X, const float *Y, int i0, int j0,
                                              int lane) {
    const int k = lane >> 4, i = lane & 15;
    f32x4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
    for (int k0 = 0; k0 < D; k0 += 4) {
        const float xa = XT ? X[(k0 + k) * LD + i0 + i] : X[(i0 + i) * LD + k0 + k];
        const float yb = YT ? Y[(j0 + i) * LD + k0 + k] : Y[(k0 + k) * LD + j0 + i];
        acc = mfma4(xa, yb, acc);
    }
    return acc;
}

// Up to 64 floats held in four separate 16-entry register vectors (unused ones
// are dead code).  vget/vput with a compile-time m fold to a plain register; with
// a wave-uniform runtime m they compile to one M0-relative register move.
typedef float vec16 __attribute__((ext_vector_type(16)));
template <int NV>
__device__ __forceinline__ float vget(const vec16 &v0, const vec16 &v1, const vec16 &v2,
                                      const vec16 &v3, int m) {
    if (NV == 1 || m < 16) return v0[m & 15];
    if (NV == 2 || m < 32) return v1[m & 15];
    if (NV == 3 || m < 48) return v2[m & 15];
    return v3[m & 15];
}
template <int NV>
__device__ __forceinline__ void vput(vec16 &v0, vec16 &v1, vec16 &v2, vec16 &v3, int m, float x) {
    if (NV == 1 || m < 16) v0[m & 15] = x;
    else if (NV == 2 || m < 32) v1[m & 15] = x;
    else if (NV == 3 || m < 48) v2[m & 15] = x;
    else v3[m & 15] = x;
}

// Moore-Penrose pseudoinverse of S = S_a + S_b, one block per pair.  A full-rank
// S is inverted directly by D pivoted symmetric sweeps; otherwise:
//  1. diagonally pivoted Cholesky, S ~ L L^T with L's rows in the original
//     order: each step takes the largest remaining diagonal of the Schur
//     complement as pivot j, column k of L is that complement's column j over
//     sqrt(pivot), and its outer product is subtracted; the factorisation stops
//     when the pivot is at or below kPivotRtol * max_i S_ii (numerical rank r);
//  2. M = L^T L (r x r, positive definite) is inverted by r symmetric sweeps
//     (the SWEEP operator keeps the matrix symmetric, so a sweep's pivot column
//     is its pivot row; after all r sweeps the block holds -M^-1);
//  3. S^+ = (L L^T)^+ = Y Y^T with Y = L M^-1 (L has full column rank).
// The working matrix lives in registers: thread t owns column c = t % D and the
// R consecutive rows d0 .. d0+R-1, d0 = (t / D) R, the same for a whole wave.
// Both the Schur complement and the swept matrix are symmetric, so a step's
// pivot column is its pivot row: the waves holding that row publish it with
// one store per lane (a wave-uniform register index), and every thread reads
// its rows' entries back as broadcasts.  Each wave keeps its own copy of the
// diagonal (lane e holds entries e, e + 64) for the pivot search, so a step
// costs one barrier.
template <int D>
__device__ __forceinline__ void pair_pinv_pivoted(const PinvArgs &a, int p, float *sm) {
    constexpr int TH = pinv_threads(D);
    constexpr int NW = TH / 64;        // waves
    constexpr int LD = D + 4;          // 16-byte rows; 16 x 4 MFMA operand reads hit 64 banks
    constexpr int NB = D / 16;
    constexpr int R = D * D / TH;     // rows per thread (16: one register vector)
    constexpr int EPL = D / 64;        // diagonal entries per lane
    constexpr int NT = NB * NB / NW;   // output tiles per wave
    float *Lt = sm;                    // [D][LD] row k = column k of L; later Y (row-major)
    float *Mb = sm + D * LD;           // [D][LD] M, later M^-1
    float *cb = Mb + D * LD;           // [2][D] published pivot row of the sweep
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar
    const int c = tid % D;
    const int d0 = __builtin_amdgcn_readfirstlane((tid / D) * R);  // wave-uniform
    const float *Sa = a.SG + (int64_t)a.pa[p] * D * D;
    const float *Sb = a.SG + (int64_t)a.pb[p] * D * D;

    // The owned rows sit in separate 16-entry register vectors: an entry picked
    // by a wave-uniform index compiles to M0-relative register moves.
    constexpr int NV = R / 16;
    vec16 A0 = {}, A1 = {}, A2 = {}, A3 = {};
#define AGET(m) vget<NV>(A0, A1, A2, A3, (m))
#define APUT(m, x) vput<NV>(A0, A1, A2, A3, (m), (x))
#pragma unroll
    for (int m = 0; m < R; ++m) {
        const int r = d0 + m;
        APUT(m, 0.5f * ((Sa[r * D + c] + Sb[r * D + c]) + (Sa[c * D + r] + Sb[c * D + r])));
    }
    float dg[EPL];
    bool ddone[EPL];
#pragma unroll
    for (int h = 0; h < EPL; ++h) {
        const int e = lane + 64 * h;
        dg[h] = Sa[e * D + e] + Sb[e * D + e];
        ddone[h] = false;
    }
    bool cdone = false;                // this thread's column already eliminated
    for (int e = tid; e < D * LD; e += TH) Lt[e] = 0.f;
    float mx = 0.f;
#pragma unroll
    for (int h = 0; h < EPL; ++h) mx = fmaxf(mx, dg[h]);
    const float stop = kPivotRtol * fkey_inv(wave_max_u32_dpp(fkey(mx)));

    auto pivot = [&](float &pv, int &j) {
        uint32_t best = 0u;
        int bi = 0;
#pragma unroll
        for (int h = 0; h < EPL; ++h) {
            const uint32_t key = ddone[h] ? 0u : fkey(dg[h]);
            if (key > best) { best = key; bi = lane + 64 * h; }
        }
        const uint32_t top = wave_max_u32_dpp(best);
        const uint64_t who = ballot(best == top);
        j = __builtin_amdgcn_readlane(bi, (int)__builtin_ctzll(who));
        pv = top ? fkey_inv(top) : -INFINITY;
    };
    float *out = a.Sp + (int64_t)p * D * D;

    // Full rank first: D symmetric sweeps of S itself, each on the largest
    // unswept diagonal entry, leave -S^-1.  The unswept diagonal is the Schur
    // complement's, so the pivots and the rank cut are those of the pivoted
    // Cholesky below; if the cut stops the sweeps early, the block starts over
    // on the rank-revealing path.
    {
        float pv;
        int j;
        pivot(pv, j);
        int swept = 0;
        for (int k = 0; k < D; ++k) {
            if (!(pv > stop)) break;   // uniform
            float *f = cb + (k & 1) * D;
            const bool own = j >= d0 && j < d0 + R;
            if (own) f[c] = AGET(__builtin_amdgcn_readfirstlane(j - d0));
            __syncthreads();
            const float ip = 1.f / f[j];
            const float fc = f[c];
            const float s = (c == j) ? 0.f : 1.f;
            const float t = (c == j) ? ip : -fc * ip;
            const float4 *fr = (const float4 *)(f + d0);
#pragma unroll
            for (int q = 0; q < R / 4; ++q) {
                const float4 v = fr[q];
                APUT(4 * q + 0, AGET(4 * q + 0) * s + v.x * t);
                APUT(4 * q + 1, AGET(4 * q + 1) * s + v.y * t);
                APUT(4 * q + 2, AGET(4 * q + 2) * s + v.z * t);
                APUT(4 * q + 3, AGET(4 * q + 3) * s + v.w * t);
            }
            if (own) APUT(__builtin_amdgcn_readfirstlane(j - d0), (c == j) ? -ip : fc * ip);
#pragma unroll
            for (int h = 0; h < EPL; ++h) {
                const float fe = f[lane + 64 * h];
                dg[h] -= fe * fe * ip;
                ddone[h] = ddone[h] || (lane + 64 * h == j);
            }
            ++swept;
            pivot(pv, j);
        }
        if (swept == D) {              // uniform
#pragma unroll
            for (int m = 0; m < R; ++m) out[(d0 + m) * D + c] = -AGET(m);
            if (tid == 0) a.rank[p] = D;
            return;
        }
    }
    // rank deficient: start over from S
#pragma unroll
    for (int m = 0; m < R; ++m) {
        const int r = d0 + m;
        APUT(m, 0.5f * ((Sa[r * D + c] + Sb[r * D + c]) + (Sa[c * D + r] + Sb[c * D + r])));
    }
#pragma unroll
    for (int h = 0; h < EPL; ++h) {
        const int e = lane + 64 * h;
        dg[h] = Sa[e * D + e] + Sb[e * D + e];
        ddone[h] = false;
    }
    __syncthreads();                   // Lt cleared; every read of the sweeps' cb is done

    float pv;
    int j;
    pivot(pv, j);
    int r = 0;
    for (int k = 0; k < D; ++k) {
        if (!(pv > stop)) break;       // uniform: every wave found the same pivot
        const float inv = __builtin_amdgcn_rsqf(pv);
        const float ljj = pv * inv;
        float *lk = Lt + k * LD;
        if (j >= d0 && j < d0 + R) {   // this wave holds row j (= column j)
            const float aj = AGET(__builtin_amdgcn_readfirstlane(j - d0));
            const float v = (c == j) ? ljj : (cdone ? 0.f : aj * inv);
            lk[c] = v;
        }
        __syncthreads();
        const float cc = lk[c];
        const float4 *cr = (const float4 *)(lk + d0);
#pragma unroll
        for (int q = 0; q < R / 4; ++q) {
            const float4 v = cr[q];
            APUT(4 * q + 0, AGET(4 * q + 0) - v.x * cc);
            APUT(4 * q + 1, AGET(4 * q + 1) - v.y * cc);
            APUT(4 * q + 2, AGET(4 * q + 2) - v.z * cc);
            APUT(4 * q + 3, AGET(4 * q + 3) - v.w * cc);
        }
#pragma unroll
        for (int h = 0; h < EPL; ++h) {
            const float ce = lk[lane + 64 * h];
            dg[h] -= ce * ce;
            ddone[h] = ddone[h] || (lane + 64 * h == j);
        }
        cdone = cdone || (c == j);
        r = k + 1;
        pivot(pv, j);
    }
    __syncthreads();

    // M = L^T L = Lt Lt^T into Mb (zero outside the leading r x r block)
    for (int t = wave; t < NB * NB; t += NW) {
        const int i0 = (t / NB) * 16, j0 = (t % NB) * 16;
        const f32x4v v = lds_tile_mm<D, LD, false, true>(Lt, Lt, i0, j0, lane);
#pragma unroll
        for (int q = 0; q < 4; ++q) Mb[(i0 + 4 * (lane >> 4) + q) * LD + j0 + (lane & 15)] = v[q];
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < R; ++m) APUT(m, Mb[(d0 + m) * LD + c]);
    // r symmetric sweeps: entry (i, c) -> A - f_i f_c / f_k off row/column k,
    // f_i / f_k in column k (and row k), -1 / f_k at (k, k), f = pivot row k
    for (int k = 0; k < r; ++k) {
        float *f = cb + (k & 1) * D;
        const bool own = k >= d0 && k < d0 + R;
        if (own) f[c] = AGET(__builtin_amdgcn_readfirstlane(k - d0));
        __syncthreads();
        const float ip = 1.f / f[k];
        const float fc = f[c];
        const float s = (c == k) ? 0.f : 1.f;
        const float t = (c == k) ? ip : -fc * ip;
        const float4 *fr = (const float4 *)(f + d0);
#pragma unroll
        for (int q = 0; q < R / 4; ++q) {
            const float4 v = fr[q];
            APUT(4 * q + 0, AGET(4 * q + 0) * s + v.x * t);
            APUT(4 * q + 1, AGET(4 * q + 1) * s + v.y * t);
            APUT(4 * q + 2, AGET(4 * q + 2) * s + v.z * t);
            APUT(4 * q + 3, AGET(4 * q + 3) * s + v.w * t);
        }
        if (own) APUT(__builtin_amdgcn_readfirstlane(k - d0), (c == k) ? -ip : fc * ip);
    }
    __syncthreads();                   // every thread is done reading Mb and cb
#pragma unroll
    for (int m = 0; m < R; ++m) Mb[(d0 + m) * LD + c] = -AGET(m);
    __syncthreads();
    // Y = L M^-1 (Y(i, c) = sum_k Lt[k][i] M^-1[k][c]); each wave keeps its tiles
    // in registers until every wave has finished reading Lt
    f32x4v y[NT];
#pragma unroll
    for (int q = 0; q < NT; ++q) {
        const int t = wave + NW * q;
        y[q] = lds_tile_mm<D, LD, true, false>(Lt, Mb, (t / NB) * 16, (t % NB) * 16, lane);
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < NT; ++q) {
        const int t = wave + NW * q;
        const int i0 = (t / NB) * 16, j0 = (t % NB) * 16;
#pragma unroll
        for (int u = 0; u < 4; ++u) Lt[(i0 + 4 * (lane >> 4) + u) * LD + j0 + (lane & 15)] = y[q][u];
    }
    __syncthreads();
    // S^+ = Y Y^T
    for (int t = wave; t < NB * NB; t += NW) {
        const int i0 = (t / NB) * 16, j0 = (t % NB) * 16;
        const f32x4v v = lds_tile_mm<D, LD, false, true>(Lt, Lt, i0, j0, lane);
#pragma unroll
        for (int q = 0; q < 4; ++q) out[(i0 + 4 * (lane >> 4) + q) * D + j0 + (lane & 15)] = v[q];
    }
    if (tid == 0) a.rank[p] = r;
#undef AGET
#undef APUT
}

// S^-1 per pair by blocked sweeps, one block per pair: rank[p] = d when S is
// comfortably full rank (S^+ = S^-1 written), else rank[p] = 0.
template <int D>
__global__ __launch_bounds__(pinv_threads(D)) void k_pair_inv(PinvArgs a) {
    extern __shared__ float sm[];
    pair_inv_blocked<D>(a, blockIdx.x, sm);
}

// (S_a + S_b)^+ by the pivoted path for the pairs k_pair_inv left (rank[p] = 0).
// Two kernels rather than one with both paths: together the paths spill, and a
// kernel with scratch memory starts its waves several microseconds later
// (measured), which would slow the common full-rank case.
template <int D>
__global__ __launch_bounds__(pinv_threads(D)) void k_pair_pinv(PinvArgs a) {
    extern __shared__ float sm[];
    if (a.rank[blockIdx.x] == D) return;  // block-uniform: k_pair_inv inverted it
    pair_pinv_pivoted<D>(a, blockIdx.x, sm);
}

// ------------------------------------------------ 4. pair loss and merge maps

struct LossArgs {
    const float *SG;     // [h_kt + P][D][D]
    const float *Sp;     // [P][D][D] (S_a + S_b)^+
    float *Pm;           // [P][2][D][D]: P_a = S_a S^+, P_b = S_b S^+
    double *part;        // [P][n_part] partial costs
    int h_kt, n_part;
    uint8_t pa[kMaxPairs], pb[kMaxPairs];
};

// C tile (i0, j0) of X Y with MFMA 16x16x4, operands (row-major D x D, global
// memory, L2/L1 resident) all loaded before the multiply chain starts.
template <int D>
__device__ __forceinline__ f32x4v tile_mm(const float *X, const float *Y, int i0, int j0, int lane) {
    const int k = lane >> 4, i = lane & 15;
    float xa[D / 4], yb[D / 4];
#pragma unroll
    for (int s = 0; s < D / 4; ++s) {
        xa[s] = X[(i0 + i) * D + 4 * s + k];
        yb[s] = Y[(4 * s + k) * D + j0 + i];
    }
    f32x4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < D / 4; ++s) acc = mfma4(xa[s], yb[s], acc);
    return acc;
}

// Tiles of the 2 (D/16)^2-tile job of one pair handled by one 4-wave block.
constexpr int kTilesPerBlock = 4;

// P_a = S_a S^+ and P_b = S_b S^+: block (pair p, tile group), one tile per wave.
template <int D>
__global__ __launch_bounds__(kThreads) void k_pair_maps(LossArgs a) {
    constexpr int NB = D / 16;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int p = blockIdx.x;
    const int t = blockIdx.y * kTilesPerBlock + wave;          // < 2 NB^2 by the grid
    const int which = t / (NB * NB), tt = t % (NB * NB);
    const int i0 = (tt / NB) * 16, j0 = (tt % NB) * 16;
    const float *S = a.SG + (int64_t)(which ? a.pb[p] : a.pa[p]) * D * D;
    const f32x4v v = tile_mm<D>(S, a.Sp + (int64_t)p * D * D, i0, j0, lane);
    float *C = a.Pm + ((int64_t)p * 2 + which) * D * D;
#pragma unroll
    for (int q = 0; q < 4; ++q) C[(i0 + 4 * (lane >> 4) + q) * D + j0 + (lane & 15)] = v[q];
}

// Partial eq. 13 costs: the pair's cost is <G P_b, P_b S_a> + <G P_a, P_a S_b>;
// block (pair p, tile group) forms one tile of both factors of one term per wave
// and writes the group's fp64 partial sum.
template <int D>
__global__ __launch_bounds__(kThreads) void k_pair_cost(LossArgs a) {
    constexpr int NB = D / 16;
    __shared__ double dsum[4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int p = blockIdx.x;
    const int t = blockIdx.y * kTilesPerBlock + wave;
    const int which = t / (NB * NB), tt = t % (NB * NB);
    const int i0 = (tt / NB) * 16, j0 = (tt % NB) * 16;
    const float *G = a.SG + (int64_t)(a.h_kt + p) * D * D;
    const float *Pm = a.Pm + ((int64_t)p * 2 + (which ? 0 : 1)) * D * D;   // term a: P_b
    const float *Sx = a.SG + (int64_t)(which ? a.pb[p] : a.pa[p]) * D * D;
    const f32x4v u = tile_mm<D>(G, Pm, i0, j0, lane);
    const f32x4v v = tile_mm<D>(Pm, Sx, i0, j0, lane);
    double part = 0.0;
#pragma unroll
    for (int q = 0; q < 4; ++q) part += (double)u[q] * (double)v[q];
    for (int o = 32; o > 0; o >>= 1) part += __shfl_xor(part, o);
    if (lane == 0) dsum[wave] = part;
    __syncthreads();
    if (threadIdx.x == 0)
        a.part[(int64_t)p * a.n_part + blockIdx.y] = (dsum[0] + dsum[1]) + (dsum[2] + dsum[3]);
}

// ------------------------------------------------------------ 5. matching

struct MatchArgs {
    const double *part;  // [P][n_part] partial pair costs
    int n_part;
    double *w;           // [h_kt][h_kt] pair costs (written here)
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
    // pair costs: fixed-order sums of the partials, mirrored, zero diagonal
    for (int p = tid; p < h * (h - 1) / 2; p += kThreads) {
        int i = 0, rest = p;
        while (rest >= h - 1 - i) { rest -= h - 1 - i; ++i; }
        const int j = i + 1 + rest;
        double L = 0.0;
        for (int q = 0; q < a.n_part; ++q) L += a.part[(int64_t)p * a.n_part + q];
        a.w[i * h + j] = L;
        a.w[j * h + i] = L;
    }
    if (tid < h) a.w[tid * h + tid] = 0.0;
    __syncthreads();
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

constexpr int kWX = 64;   // output columns x per block (d_model is a multiple of 64)
constexpr int kWC = 16;   // merged channels per block

// out row i*D + c, column x = sum_e W[a*D+e][x] P_a[e][c] + W[b*D+e][x] P_b[e][c]
// (eq. 15 in the weight layout: merged head i = pair (a, b) = pairs[i]).  Block
// (i, kWC channels, kWX columns): the two heads' weight rows over the block's
// columns and the channels' columns of P_a and P_b are staged in LDS with
// 16-byte loads; thread (x, channel quad) accumulates four channels of column x.
template <int D>
__global__ __launch_bounds__(kThreads) void k_merged_weight(WeightArgs a) {
    static_assert(kThreads == kWX * kWC / 4, "one thread per column and channel quad");
    __shared__ uint16_t wsl[2][D][kWX];
    __shared__ float psl[2][D][kWC];
    const int tid = threadIdx.x;
    const int hi = blockIdx.x, c0 = blockIdx.y * kWC, x0 = blockIdx.z * kWX;
    const int ia = a.pairs[2 * hi], ib = a.pairs[2 * hi + 1];
    if (ia < 0 || ib <= ia || ib >= a.h_kt) return;      // uniform per block
    const int p = ia * (2 * a.h_kt - ia - 1) / 2 + (ib - ia - 1);
    const float *src = a.Pm + (int64_t)p * 2 * D * D;
    constexpr int W8 = kWX / 8;                           // 16-byte pieces of a staged row
    for (int e = tid; e < 2 * D * W8; e += kThreads) {
        const int h = e / (D * W8), r = (e / W8) % D, k8 = e % W8;
        const uint16_t *g = a.W + ((int64_t)(h ? ib : ia) * D + r) * a.dm + x0 + 8 * k8;
        *(u32x4 *)&wsl[h][r][8 * k8] = ld16(g);
    }
    constexpr int P4 = kWC / 4;
    for (int e = tid; e < 2 * D * P4; e += kThreads) {
        const int h = e / (D * P4), r = (e / P4) % D, c4 = e % P4;
        *(float4 *)&psl[h][r][4 * c4] = *(const float4 *)(src + h * D * D + r * D + c0 + 4 * c4);
    }
    __syncthreads();
    const int x = tid % kWX, cq = tid / kWX;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
    for (int e = 0; e < D; ++e) {
        const float va = __uint_as_float((uint32_t)wsl[0][e][x] << 16);
        const float vb = __uint_as_float((uint32_t)wsl[1][e][x] << 16);
        const float4 pa = *(const float4 *)&psl[0][e][4 * cq];
        const float4 pb = *(const float4 *)&psl[1][e][4 * cq];
        acc[0] += va * pa.x + vb * pb.x;
        acc[1] += va * pa.y + vb * pb.y;
        acc[2] += va * pa.z + vb * pb.z;
        acc[3] += va * pa.w + vb * pb.w;
    }
    float *o = a.out + (int64_t)(hi * D + c0 + 4 * cq) * a.dm + x0 + x;
#pragma unroll
    for (int c = 0; c < 4; ++c) o[(int64_t)c * a.dm] = acc[c];
}

}  // namespace merge
}  // namespace saga
