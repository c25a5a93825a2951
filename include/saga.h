/*
 * saga.h -- C ABI of the SAGA + Atop-N sparse decode-attention library for
 * AMD Instinct MI355X (gfx950).
 *
 * The method ("More Value per Key: Asymmetric Sparse Attention for Faster
 * LLM Decoding", picx.dev summary):
 *   - scores A = q K^T / sqrt(d) over h_k key heads        (eqs. 2-4)
 *   - keep the entries of each score row with A >= tau,     (Methodology >
 *     tau being the row's N-th largest score                 Atop-N, item 1;
 *                                                            eq. 6)
 *   - tau recomputed exactly once every R decode steps      (Atop-N, item 2)
 *     and reused in between
 *   - O = softmax(A[S]) V[S] over the survivors S, read     (Atop-N, eq. 7;
 *     from h_v value heads, h_k <= h_v <= h_q                SAGA Architecture)
 * Head map (the pages give none; this library's reading): query head j
 * reads key head floor(j*h_k/h_q) and value head floor(j*h_v/h_q).
 *
 * Conventions for every entry point below:
 *   - Tensor pointers are DEVICE pointers owned by the caller, contiguous,
 *     16-byte aligned.  Layouts (row-major, innermost last):
 *       Q   bf16  [B][h_q][d]          one decode step's queries
 *       K   bf16  [B][h_k][l_kv][d]    key cache   (h_kv heads for dense)
 *       V   bf16  [B][h_v][l_kv][d]    value cache (h_kv heads for dense)
 *       tau fp32  [B][h_q]             per-row threshold (same units as A)
 *       O   fp32  [B][h_q][d]          attention output
 *       counts int32 [B][h_q]          |S| per row
 *   - ws / ws_bytes: caller-owned device workspace of at least the size the
 *     matching *_workspace_bytes() call returns.  Before its first use a
 *     workspace must be cleared once with saga_workspace_init(); every call
 *     leaves its internal counters back at zero, so no further clearing is
 *     needed.  Calls that share one workspace must not overlap in time
 *     (use one workspace per stream).
 *   - hip_stream: a hipStream_t (NULL = the default stream).  All work is
 *     enqueued asynchronously; the library never allocates, frees or
 *     synchronizes.
 *   - Arguments are validated on the host before anything is enqueued; an
 *     invalid call returns a negative saga_status and enqueues nothing.
 *     Launch failures are reported as SAGA_ERR_HIP.
 *   - Supported: d in {64, 128}; 1 <= h_k <= h_v <= h_q <= 32768; h_q/h_k
 *     rounded up <= 64; 1 <= N <= l_kv; l_kv * d * 2 < 2^31; B*h_q < 2^20.
 */
#ifndef SAGA_H
#define SAGA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum saga_status {
    SAGA_OK = 0,
    SAGA_ERR_INVALID_ARG = -1, /* null/misaligned pointer, inconsistent sizes */
    SAGA_ERR_UNSUPPORTED = -2, /* valid for the method but outside the supported shapes */
    SAGA_ERR_WORKSPACE = -3,   /* ws_bytes smaller than required */
    SAGA_ERR_HIP = -4          /* a HIP launch or runtime call failed */
} saga_status;

/* Human-readable name of a status code (static string, never NULL). */
const char *saga_status_string(int status);

/* Library ABI version (major*10000 + minor*100 + patch). */
int saga_version(void);

/* Bytes of workspace saga_decode_step / saga_refresh_threshold need for this
 * shape (0 when the shape is invalid or unsupported).  Pure host function. */
size_t saga_workspace_bytes(int B, int h_q, int h_k, int h_v, int d, int64_t l_kv, int64_t N);

/* Bytes of workspace saga_dense_gqa_baseline needs (0 when invalid). */
size_t saga_dense_workspace_bytes(int B, int h_q, int h_kv, int d, int64_t l_kv);

/* Zero the workspace's internal counters (enqueued on hip_stream with a fill
 * kernel, so it may be captured in a HIP graph).  Call once per workspace. */
int saga_workspace_init(void *ws, size_t ws_bytes, void *hip_stream);

/*
 * Exact threshold refresh (Atop-N item 2; eq. 6):
 *   tau[b][j] := the N-th largest of A[b][j][0..l_kv), A = q K^T / sqrt(d)
 * computed in fp32 (bf16 products, fp32 accumulation, -0 canonicalised to
 * +0), i.e. element N-1 of the row sorted in descending order, ties kept.
 * The fp32 scores are left in the workspace (see saga_workspace_layout).
 */
int saga_refresh_threshold(const void *Q, const void *K, int B, int h_q, int h_k, int d,
                           int64_t l_kv, int64_t N, float *tau, void *ws, size_t ws_bytes,
                           void *hip_stream);

/*
 * One Atop-N decode step (Atop-N items 1-2, eq. 7):
 *   if refresh != 0: tau is first recomputed from this step's scores exactly
 *                    as saga_refresh_threshold does (tau is then an output);
 *   S[b][j]   := { t : A[b][j][t] >= tau[b][j] }  (no cap on |S|);
 *   O[b][j]   := sum_{t in S} softmax_S(A[b][j])_t * V[b][vh(j)][t]  (fp32),
 *                or all zeros when S is empty;
 *   counts[b][j] := |S|  (counts may be NULL).
 * N is the row rank the refresh selects and sizes internal buffers.
 */
int saga_decode_step(const void *Q, const void *K, const void *V, int B, int h_q, int h_k,
                     int h_v, int d, int64_t l_kv, int64_t N, float *tau, int refresh, float *O,
                     int32_t *counts, void *ws, size_t ws_bytes, void *hip_stream);

/*
 * The two halves of saga_decode_step, for callers that want the selection on
 * its own or time the stages separately.  saga_decode_step(...) is exactly
 * saga_select(...) followed by saga_attend(...) on the same workspace.
 *
 * saga_select: (refresh as in saga_decode_step) scores, compare with tau and
 *   compact the survivors S into the workspace's segment records (layout
 *   below).
 * saga_attend: O and counts from the records the preceding saga_select on
 *   this workspace left, for the same shape (eq. 7).
 */
int saga_select(const void *Q, const void *K, int B, int h_q, int h_k, int h_v, int d,
                int64_t l_kv, int64_t N, float *tau, int refresh, void *ws, size_t ws_bytes,
                void *hip_stream);

int saga_attend(const void *V, int B, int h_q, int h_k, int h_v, int d, int64_t l_kv, int64_t N,
                float *O, int32_t *counts, void *ws, size_t ws_bytes, void *hip_stream);

/*
 * saga_decode_step with a cheaper exact refresh.  pivot: caller-owned int32
 * device array [B*h_q][N], the per-row state of this refresh scheme (like
 * tau, one per layer / sequence), written by every refresh.
 *   refresh 0: compare with tau, as saga_decode_step; pivot is not touched.
 *   refresh 1: exact refresh as saga_decode_step, then N positions of each
 *              row's survivors are recorded in pivot (increasing).
 *   refresh 2: exact refresh from pivot: the least current score over the
 *              row's N recorded positions, less a rounding margin, is a lower
 *              bound on the new N-th largest score; one compare pass lists
 *              every score at or above it and the exact N-th largest is
 *              selected among those (same tau as refresh 1, bit for bit);
 *              the new survivors' positions are recorded again.  A pivot row
 *              that is not N strictly increasing positions inside the cache
 *              gives the bound -inf: still exact, but it lists every score.
 * The threshold refresh is defined in Methodology > Atop-N Attention (items
 * 1-2, eq. 6) of the pages; this entry point only changes how it is found.
 */
int saga_decode_step_pivot(const void *Q, const void *K, const void *V, int B, int h_q, int h_k,
                           int h_v, int d, int64_t l_kv, int64_t N, float *tau, int32_t *pivot,
                           int refresh, float *O, int32_t *counts, void *ws, size_t ws_bytes,
                           void *hip_stream);

/*
 * Dense full-attention GQA decode, the in-run baseline (eqs. 2-4):
 *   O[b][j] := softmax(q K_g^T / sqrt(d)) V_g,  g = floor(j*h_kv/h_q),
 * with K, V both [B][h_kv][l_kv][d] bf16; fp32 output.
 */
int saga_dense_gqa_baseline(const void *Q, const void *K, const void *V, int B, int h_q,
                            int h_kv, int d, int64_t l_kv, float *O, void *ws, size_t ws_bytes,
                            void *hip_stream);

/*
 * A growing context: caches with room for cap rows per head, K bf16
 * [B][h_k][cap][d] and V bf16 [B][h_v][cap][d], of which the first len rows
 * hold the context (the decode step just before the method's: each new
 * token's key and value rows are appended, and the new key is compared with
 * the stale tau like every other position; Methodology > Atop-N Attention,
 * item 2).
 *
 * saga_append_kv: K[b][g][pos] := k_new[b][g], V[b][v][pos] := v_new[b][v]
 *   (k_new bf16 [B][h_k][d], v_new bf16 [B][h_v][d]); 0 <= pos < cap.
 * saga_decode_step_cache: saga_decode_step_pivot over the first len rows
 *   (N <= len <= cap).  ws: saga_cache_workspace_bytes(.., cap, N) bytes,
 *   valid for every len <= cap.  The pivot rows are positions in the record
 *   order of the chunking for len; when growth changes the chunking (about
 *   every 64 * 256 / (B * h_k) rows) the next refresh from the pivot lists
 *   every position: exact, slower.
 */
size_t saga_cache_workspace_bytes(int B, int h_q, int h_k, int h_v, int d, int64_t cap, int64_t N);
int saga_append_kv(void *K, void *V, const void *k_new, const void *v_new, int B, int h_k,
                   int h_v, int d, int64_t cap, int64_t pos, void *hip_stream);
int saga_decode_step_cache(const void *Q, const void *K, const void *V, int B, int h_q, int h_k,
                           int h_v, int d, int64_t cap, int64_t len, int64_t N, float *tau,
                           int32_t *pivot, int refresh, float *O, int32_t *counts, void *ws,
                           size_t ws_bytes, void *hip_stream);

/*
 * SAGA full attention: the decoupled heads without the sparsity, softmax
 * over every cache position (SAGA Architecture; eqs. 2-4 with key head
 * floor(j*h_k/h_q) and value head floor(j*h_v/h_q)):
 *   O[b][j] := softmax(q_j K_{kh(j)}^T / sqrt(d)) V_{vh(j)},
 * K bf16 [B][h_k][l_kv][d], V bf16 [B][h_v][l_kv][d], 1 <= h_k <= h_v <= h_q,
 * d in {64, 128}; fp32 output [B][h_q][d].  Each key row is read once per
 * key head (once per subset of four value heads when a key head serves more
 * than four), each value row once.  ws: saga_full_attention_workspace_bytes
 * bytes, 256-byte aligned.  h_k = h_v is saga_dense_gqa_baseline.  Returns
 * SAGA_ERR_UNSUPPORTED when a block would serve more than 16 query heads.
 */
size_t saga_full_attention_workspace_bytes(int B, int h_q, int h_k, int h_v, int d, int64_t l_kv);
int saga_full_attention(const void *Q, const void *K, const void *V, int B, int h_q, int h_k,
                        int h_v, int d, int64_t l_kv, float *O, void *ws, size_t ws_bytes,
                        void *hip_stream);

/*
 * saga_decode_step_pivot without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The workspace is a static array inside
 * the library, one per GPU, of SAGA_STATIC_WORKSPACE_BYTES bytes (128 MiB),
 * held from the library's first use on that GPU until the process ends; this
 * entry point itself allocates nothing.  Shapes whose workspace
 * (saga_workspace_bytes) exceeds it return SAGA_ERR_WORKSPACE and enqueue
 * nothing; the 128K-context Llama-3.2-1B shape needs 65 MiB, the batch-4
 * Qwen2.5-1.5B shape 97 MiB.  Every call on one GPU shares that GPU's array:
 * calls that overlap in time on one GPU (several streams or host threads)
 * race and must be serialised by the caller.  Results equal
 * saga_decode_step_pivot's bit for bit.  The array's device address is looked
 * up once per device, on the first call made with that device current.
 */
#define SAGA_STATIC_WORKSPACE_BYTES (128u << 20)
int saga_decode_step_noalloc(const void *Q, const void *K, const void *V, int B, int h_q, int h_k,
                             int h_v, int d, int64_t l_kv, int64_t N, float *tau, int32_t *pivot,
                             int refresh, float *O, int32_t *counts, void *hip_stream);

/* Where the last call left its intermediate results inside the workspace
 * (byte offsets from ws), for inspection and testing. */
typedef struct saga_ws_layout {
    size_t bytes;          /* total workspace size (= saga_workspace_bytes) */
    size_t scores_off;     /* fp32 [B*h_q][scores_ld]: scores of the last refresh */
    int64_t scores_ld;     /* row stride of the scores, in elements (>= l_kv) */
    size_t seg_off;        /* int32 [B*h_q][n_seg][seg_words]: survivor records, each
                              { count, order key of the max score, then (t, score bits)
                              pairs }; segment k = 4c + s of a row lists positions of
                              chunk c from its groups of seg_group rows s, s+8, s+16,
                              ..., then s+4, s+12, ... (seg_cap positions in all) */
    int64_t seg_words;     /* int32 words per record (multiple of 16) */
    int64_t chunk_len;     /* cache positions per streaming block */
    int64_t n_chunk;       /* blocks per key-head row: ceil(l_kv / chunk_len) */
    int64_t n_seg;         /* segments per row (n_chunk * 4) */
    int64_t seg_cap;       /* positions covered by one segment (chunk_len / 4) */
    int64_t seg_group;     /* rows per group of a segment: 16 times the select pass's
                              tiles per wave iteration (16: one tile) */
} saga_ws_layout;

/* Fill *out for this shape.  Returns SAGA_OK or a negative status. */
int saga_workspace_layout(int B, int h_q, int h_k, int h_v, int d, int64_t l_kv, int64_t N,
                          saga_ws_layout *out);

/*
 * Expand the survivor segments of the last saga_decode_step (or
 * saga_decode_step_pivot) on this workspace into a byte mask: mask[b][j][t]
 * = 1 if t was in S[b][j], else 0.  mask is a device pointer of B*h_q*l_kv
 * bytes.  Enqueued on hip_stream.
 */
int saga_selection_mask(const void *ws, size_t ws_bytes, int B, int h_q, int h_k, int h_v, int d,
                        int64_t l_kv, int64_t N, uint8_t *mask, void *hip_stream);

/*
 * Measurement utility, not part of the method: read the `bytes` bytes at buf
 * once with the streaming kernels' launch shape (256 workgroups of 8 waves,
 * 16-byte non-temporal loads, eight in flight per lane) and store, for each
 * workgroup i, the XOR of the 32-bit words it read in sink[i].  Its rate is
 * the achievable-read reference the streaming kernels are compared with.
 * buf: device pointer, 16-byte aligned, bytes a positive multiple of 16;
 * sink: device array of SAGA_PROBE_SINK_WORDS words (entries past the
 * workgroups used are left untouched).  Enqueued on hip_stream.
 */
#define SAGA_PROBE_SINK_WORDS 256
int saga_read_probe(const void *buf, int64_t bytes, uint32_t *sink, void *hip_stream);

/*
 * Measurement utility, not part of the method: the same plain read with a
 * chosen launch shape, for finding the fastest cold read of a buffer on this
 * GPU.  blocks (1..65536) workgroups of `waves` waves (4 or 8), `loads`
 * 16-byte non-temporal loads in flight per lane (4, 8 or 16 with 4 waves; 4
 * or 8 with 8 waves, else SAGA_ERR_UNSUPPORTED).  chunked != 0: workgroup i
 * reads the i-th of `blocks` contiguous ranges; chunked == 0: the workgroups
 * take consecutive runs of waves*64*loads items in turn.  Workgroup i XORs
 * the words it read into sink[i % SAGA_PROBE_SINK_WORDS] (so the XOR of the
 * whole sink, cleared beforehand, is the XOR of every word of the buffer).
 */
int saga_read_probe_shape(const void *buf, int64_t bytes, int blocks, int waves, int loads,
                          int chunked, uint32_t *sink, void *hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* SAGA_H */
