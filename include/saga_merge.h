/*
 * saga_merge.h -- C ABI of the GQA -> SAGA key-head merge (conversion, Stage 1)
 * for AMD Instinct MI355X (gfx950).  Part of libsaga.so; status codes and
 * stream/workspace conventions are those of saga.h.
 *
 * The method ("More Value per Key: Asymmetric Sparse Attention for Faster
 * LLM Decoding", picx.dev summary, GQA-to-SAGA Conversion, Stage 1):
 *   - a GQA teacher with h_kt key heads becomes a SAGA student with h_kt/2
 *     key heads by merging teacher heads in pairs (a, b);
 *   - the merged key projection of a pair is eq. 15 (Lemma 4.1):
 *       W_hat(a,b) = (W_a S_a + W_b S_b)(S_a + S_b)^+,
 *     S_r = sum over the query heads j of group r of Q_j^T Q_j, "+" the
 *     Moore-Penrose pseudoinverse;
 *   - a pair's cost is eq. 13 at that projection: the squared error of the
 *     logits Q_j (X W)^T of both groups' query heads over the calibration
 *     tokens;
 *   - the pairing minimises the summed cost (eq. 14); Theorem 4.2: it is a
 *     minimum-weight perfect matching on the complete graph of pair costs.
 * Readings of this library (the pages leave them open):
 *   - group r = the query heads j with floor(j*h_kt/h_q) == r (the GQA map);
 *   - the pseudoinverse's numerical rank is the number of pivots, taken on
 *     the largest remaining Schur-complement diagonal of S_a + S_b, before
 *     that diagonal falls to 2^-14 times the largest diagonal entry of S; at
 *     full rank S^+ = S^-1, else with S = L L^T at that rank (pivoted
 *     Cholesky) S^+ = L (L^T L)^-2 L^T (fp32 arithmetic; a spectrum with no
 *     gap near that level makes the result depend on rounding).  S^-1 is
 *     first formed without pivoting and kept when 1/trace(S^-1) is at least
 *     4 times that cut (every pivot then clears it); otherwise the pair takes
 *     the pivoted path;
 *   - equal-cost pairings: the one whose lowest head takes the lowest
 *     partner wins, recursively;
 *   - merged head i serves the query heads of teacher groups pairs[i][0]
 *     and pairs[i][1] (the student's query heads are those groups, in
 *     that order).
 *
 * Layouts (device pointers, row-major, 16-byte aligned, caller-owned):
 *   X        bf16  [n][d_model]        calibration inputs of the layer
 *   Q        bf16  [n][h_q][d]         calibration queries (Q_j = Q[:, j, :])
 *   W_K      bf16  [h_kt*d][d_model]   teacher key projection as a linear-layer
 *                                      weight: keys = X W_K^T, head r is rows
 *                                      r*d .. r*d+d-1 (the pages' W_K^r is the
 *                                      transpose of that block)
 *   W_merged fp32  [h_kt/2*d][d_model] merged projection, same layout
 *   pairs    int32 [h_kt/2][2]         pairs[i] = {a, b}, a < b, sorted by a
 *   pair_loss fp64 [h_kt][h_kt]        eq. 13 cost of every pair (symmetric,
 *                                      zero diagonal)
 *   total_loss fp64 [1]                summed cost of the pairing
 * Arithmetic: keys X W_K^T from bf16 products accumulated in fp32; second
 * moments of the queries from exact bf16 products, of the fp32 key
 * differences from a bf16 high/low split (about 2^-16 relative), both summed
 * in fp32 per block and fp64 across blocks; the pseudoinverse (blocked
 * symmetric sweeps, or pivoted Cholesky and symmetric sweeps inverting
 * L^T L) and the d x d products in fp32;
 * costs summed in fp64.
 * Supported: d in {64, 128}; h_kt even, 2 <= h_kt <= 16; h_kt <= h_q <= 1024;
 * d_model a multiple of 64, 64 <= d_model <= 32768; 1 <= n <= 2^26.
 */
#ifndef SAGA_MERGE_H
#define SAGA_MERGE_H

#include <stddef.h>
#include <stdint.h>

#include "saga.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes of workspace saga_merge_key_heads needs (0 when the shape is invalid
 * or unsupported).  About n*h_kt*d*4 bytes for the projected keys plus a few
 * MB of per-block partial sums and per-pair matrices.  Pure host function. */
size_t saga_merge_workspace_bytes(int64_t n, int h_q, int h_kt, int d, int d_model);

/*
 * GQA -> SAGA closed-form key merge (eqs. 13-15, Theorem 4.2):
 *   pair_loss[a][b] := eq. 13 at the eq. 15 merge of teacher heads a and b,
 *   pairs           := the minimum-weight perfect matching of pair_loss
 *                      (or pairs_in, when given),
 *   total_loss[0]   := sum of pair_loss over pairs,
 *   W_merged rows i*d .. i*d+d-1 := eq. 15 for pairs[i], in the W_K layout.
 * pairs_in: HOST array [h_kt/2][2] of a caller-chosen pairing (every head
 * exactly once, any order within and across pairs), or NULL to optimise.
 * The workspace needs no initialisation (saga_workspace_init is not
 * required); every call overwrites what it uses.
 * Errors: SAGA_ERR_INVALID_ARG for null or misaligned pointers, n < 1 or a
 * pairs_in that is not a perfect matching of 0..h_kt-1; SAGA_ERR_UNSUPPORTED
 * for shapes outside the supported set; SAGA_ERR_WORKSPACE when ws_bytes is
 * too small; SAGA_ERR_HIP if a launch fails.  Nothing is enqueued on error.
 */
int saga_merge_key_heads(const void *X, const void *Q, const void *W_K, int64_t n, int h_q,
                         int h_kt, int d, int d_model, const int32_t *pairs_in, float *W_merged,
                         int32_t *pairs, double *pair_loss, double *total_loss, void *ws,
                         size_t ws_bytes, void *hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* SAGA_MERGE_H */
