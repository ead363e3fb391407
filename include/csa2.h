/*
 * csa2.h — C ABI of the MI355X (gfx950) CSA2 hot-path library (libcsa2.so).
 *
 * CSA2 (Compressed Sparse Attention 2) is the global-attention step of
 * DeepSeek-V4.1-Flash ("DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache
 * Compression", sec. 2.3).  Per query it (1) scores every causally visible
 * compressed entry with a lightweight indexer, (2) keeps the top-k entries,
 * (3) gathers those entries from an FP4 main-KV cache and dequantises them,
 * and (4) runs shared-key/value multi-head attention over them together with
 * the layer's sliding-window (SWA) KV in one softmax.  A Reuse-mode layer
 * (sec. 2.3.1) repeats (3)-(4) with its own query and window over the index
 * list and KV published by an earlier layer.
 *
 * Fixed shapes (sec. 4.2.1 of the report): 32 indexer heads of dim 128,
 * top-k 512, 64 query heads of dim 512, window n_win <= 128.
 *
 * Conventions for every entry point
 *  - All tensor pointers are DEVICE pointers, owned by the caller, row-major,
 *    16-byte aligned.  The library never allocates, frees or retains them;
 *    scratch memory comes only from the caller's workspace.
 *  - bf16 tensors are passed as void* holding IEEE bfloat16 bit patterns.
 *  - Queries are grouped by sequence: query t belongs to sequence
 *    b = t / q_per_seq, and T = B * q_per_seq.  Decode uses q_per_seq = 1;
 *    a prefill chunk of one sequence uses B = 1, q_per_seq = T.
 *  - Causal visibility: with compression ratio m, compressed entry j covers
 *    tokens [m*j, m*j+m) and is visible to the token at absolute position p
 *    iff m*(j+1) <= p+1, so n_vis(t) = min(N, floor((q_pos[t]+1)/m)); a
 *    negative position sees no entry.  q_pos == NULL means every one of the
 *    N entries is visible.
 *  - hip_stream is a hipStream_t (e.g. torch.cuda.current_stream().cuda_stream);
 *    NULL means the default stream.  Calls only enqueue work and return.
 *  - Errors: arguments are checked on the host before anything is launched;
 *    on any error nothing is enqueued and the status says why.  Device data
 *    (positions, indices, window ends) is never read on the host: values out
 *    of the documented ranges give undefined results.  Device faults surface
 *    at the caller's next synchronisation.
 *  - Thread safety: no global mutable state; calls on different streams with
 *    disjoint outputs and workspaces may run concurrently.
 */
#ifndef CSA2_H
#define CSA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA2_IDX_HEADS 32
#define CSA2_IDX_DIM 128
#define CSA2_HEADS 64
#define CSA2_DIM 512
#define CSA2_TOPK 512
#define CSA2_MAX_WINDOW 128
#define CSA2_MAX_LAYERS 8
#define CSA2_FP4_ROW_BYTES 256   /* 512 E2M1 codes, element 2i in the low nibble of byte i */
#define CSA2_FP4_SCALES 16       /* E8M0 scale bytes per entry, one per 32 channels */

typedef enum {
    CSA2_OK = 0,
    CSA2_ERR_INVALID_ARG = 1,  /* null/misaligned pointer, non-positive size, bad scale */
    CSA2_ERR_UNSUPPORTED = 2,  /* k != 512, window or layer count out of range, size limits */
    CSA2_ERR_WORKSPACE = 3,    /* workspace pointer NULL or smaller than required */
    CSA2_ERR_LAUNCH = 4        /* the HIP runtime rejected a kernel launch */
} csa2_status;

/* Human-readable name of a status code (static string). */
const char* csa2_status_string(int32_t status);
/* Library version string, e.g. "csa2-mi355x 0.1 gfx950". */
const char* csa2_version(void);

/* ------------------------------------------------------------------ index
 * Indexer scan: for each query t and each visible entry s < n_vis(t),
 *   I(t,s) = sum_{h<32} w[t][h] * ReLU( sum_{c<128} q_idx[t][h][c] * k_idx[b][s][c] )
 * (lightning-indexer score of DeepSeek-V4, gzher.com reading sec. 4.1, which
 * CSA2 keeps, report sec. 2.3).  The scores are computed with bf16 MFMA and
 * fp32 accumulation.  Entries are grouped in tiles of CSA2_TILE consecutive
 * indices; the selection (csa2_topk) needs only each tile's maximum score and
 * re-derives the scores of the few tiles that can hold a top-k entry, so the
 * full score matrix is an optional output.
 *
 *  q_idx     bf16  [T][32][128]   indexer queries
 *  w_idx     fp32  [T][32]        per-head indexer weights
 *  k_idx     bf16  [B][N][128]    indexer keys (B = T / q_per_seq)
 *  q_pos     int32 [T] or NULL    absolute token positions (see visibility)
 *  ratio     compression ratio m >= 1
 *  scores    fp32  [T][N] out, or NULL:  I(t,s) for s < n_vis(t), -inf beyond
 *  tile_max  fp32  [T][ld] out, ld = csa2_tile_max_ld(N) = 4 * ceil(N / 64):
 *            tile_max[t][j] = max of the scores of entries 16j .. 16j+15 (those
 *            < N), -inf if none of them is visible; the ld - ceil(N/16)
 *            padding slots of each row are left unspecified
 *  stats     uint32 out, csa2_index_stats_bytes(T, q_per_seq, N) bytes: the
 *            summary the selection consumes.  Its first T * CSA2_STATS_WORDS
 *            words are a header per query that the scan sets to zero and
 *            csa2_topk fills (see there); the rest (maxima of disjoint groups
 *            of each query's entries, partial maxima of ||K_s||^2 per
 *            group of queries of a sequence) has no documented layout.
 *  stats_bytes  size of stats; smaller than csa2_index_stats_bytes -> INVALID_ARG
 * The call is one kernel and uses no workspace.
 * Requires T >= 1, q_per_seq >= 1, T % q_per_seq == 0, 1 <= N < 2^31
 * (csa2_index_stats_bytes returns 0 otherwise).
 */
#define CSA2_TILE 16
#define CSA2_STATS_WORDS 4
int64_t csa2_tile_max_ld(int64_t N);
size_t csa2_index_stats_bytes(int32_t T, int32_t q_per_seq, int64_t N);
csa2_status csa2_index(const void* q_idx, const float* w_idx, const void* k_idx,
                       const int32_t* q_pos, int32_t ratio, int32_t T, int32_t q_per_seq, int64_t N,
                       float* scores, float* tile_max, uint32_t* stats, size_t stats_bytes,
                       void* hip_stream);

/* ------------------------------------------------------------------- topk
 * Exact top-k: for each query, the first min(k, n_vis) entries of the order
 * (I_fp64 descending, index ascending) — I_fp64 as defined under csa2_index —
 * written ASCENDING by entry index into indices[t][0..], the remaining slots
 * set to -1 (report sec. 2.3: each query keeps its top-k entries; k = 512 per
 * sec. 4.2.1).  The fp32 scores only pick the candidates; the final order is
 * decided on fp64 scores computed on the device, so the result does not
 * depend on MFMA rounding.
 *
 *  scores     the scores output of csa2_index, or NULL.  When given and
 *             N <= CSA2_TOPK_ROW_MAX, each query's row is selected in LDS in one
 *             pass; otherwise the selection works from tile_max and the keys,
 *             and when given it reads the fp32 scores of the candidate tiles
 *             from the matrix (64 bytes per tile) instead of re-deriving them
 *             from the keys (4 KiB per tile).  Writing the matrix slows the
 *             scan by more than this saves at the decode shapes measured, so
 *             it pays only where the matrix exists anyway.  The indices are
 *             the same either way.
 *  tile_max, stats, stats_bytes   outputs of csa2_index for the same
 *             arguments (T, q_per_seq, N as passed to it).  For every query
 *             csa2_topk writes into the stats header:
 *             [0] eps_t (fp32 bits) >= |score(t,s) - I_fp64(t,s)| for every
 *                 visible s, where score is csa2_index's fp32 score and I_fp64
 *                 the score evaluated in fp64 with one fma per term, channels
 *                 then heads in order;
 *             [1] floor_t (fp32 bits; tile regime only, the row regime leaves
 *                 the word as csa2_index wrote it): at least CSA2_TOPK visible
 *                 entries have fp32 score >= floor_t (-inf when fewer than
 *                 CSA2_TOPK of the maxima it ranks are finite);
 *             [2], [3] counters, used and left zero (concurrent csa2_topk
 *                 calls must not share a stats array).
 *             Every candidate of the selection has fp32 score >= floor - 2 eps.
 *  q_idx, w_idx, k_idx, q_pos, ratio   as passed to csa2_index
 *  k          must be CSA2_TOPK (512)
 *  indices    int32 [T][k] out
 *  workspace >= csa2_topk_workspace_bytes(T, N, k).  A larger workspace only
 *  raises the number of candidates handled on the fast path; a smaller one
 *  (down to csa2_topk_min_workspace_bytes) is accepted and falls back to a
 *  slower exact streaming path when the candidates do not fit.
 */
#define CSA2_TOPK_ROW_MAX 36864
size_t csa2_topk_workspace_bytes(int32_t T, int64_t N, int32_t k);
size_t csa2_topk_min_workspace_bytes(int32_t T, int64_t N, int32_t k);
csa2_status csa2_topk(const float* scores, const float* tile_max, uint32_t* stats, size_t stats_bytes,
                      const void* q_idx, const float* w_idx, const void* k_idx, const int32_t* q_pos,
                      int32_t ratio, int32_t T, int32_t q_per_seq, int64_t N, int32_t k, int32_t* indices,
                      void* workspace, size_t workspace_bytes, void* hip_stream);

/* ------------------------------------------------------ selection order
 * csa2_topk_ex / csa2_topk_mxfp4_ex: csa2_topk / csa2_topk_mxfp4 with a
 * choice of the order the k entries are taken in.
 *  CSA2_SELECT_EXACT  (I_fp64 descending, index ascending): csa2_topk.
 *  CSA2_SELECT_BF16   (bf16(I_fp64) descending, index ascending), where bf16()
 *                     is rounding to the nearest bf16 value, ties to the even
 *                     significand (quantum 2^-133 below 2^-126).  The
 *                     gzher.com DeepSeek-V4 reading (FP4 QAT section) states
 *                     that the index scores are quantised to BF16 before the
 *                     top-k selector; entries whose scores round to the same
 *                     bf16 value tie, and the lower index wins.
 * Any other value of select returns CSA2_ERR_UNSUPPORTED; all other arguments,
 * outputs, workspace and errors are those of csa2_topk (csa2_topk_mxfp4).
 */
#define CSA2_SELECT_EXACT 0
#define CSA2_SELECT_BF16 1
csa2_status csa2_topk_ex(const float* scores, const float* tile_max, uint32_t* stats, size_t stats_bytes,
                         const void* q_idx, const float* w_idx, const void* k_idx, const int32_t* q_pos,
                         int32_t ratio, int32_t T, int32_t q_per_seq, int64_t N, int32_t k, int32_t select,
                         int32_t* indices, void* workspace, size_t workspace_bytes, void* hip_stream);

/* --------------------------------------------------------------- hsi pool
 * Candidate pool of the hierarchical sparse indexer (report sec. 2.3.2; block
 * size 8 and 2048 blocks per sec. 4.2.1).  A Full layer's visible entries
 * are cut into aligned blocks of CSA2_HSI_BLOCK; a block's score is the
 * largest I_fp64 (as under csa2_index) of its visible entries.  The first
 * min(CSA2_HSI_BLOCKS, number of visible blocks) blocks of the order (block
 * score descending, block index ascending) are kept, and their visible
 * entries, ascending, are written to pool[t][0..]; the remaining slots are
 * set to -1.  A query with at most CSA2_HSI_POOL visible entries keeps all of
 * them.  Later Reindex layers select their own top-k within the pool.
 *
 *  tile_max, stats, stats_bytes   outputs of csa2_index for the same
 *             arguments (read only; the header words are not touched)
 *  q_idx, w_idx, k_idx, q_pos, ratio, T, q_per_seq, N   as passed to csa2_index
 *  pool       int32 [T][CSA2_HSI_POOL] out
 *  workspace >= csa2_hsi_pool_workspace_bytes(T, N); its first 16*T bytes
 *             hold {eps_t, floor_t, 0, 0} per query afterwards (as the stats
 *             header of csa2_topk, with floor_t ranking CSA2_HSI_BLOCKS
 *             distinct blocks)
 *  Three kernels; requires 1 <= N < 2^31, T <= 65535.
 */
#define CSA2_HSI_BLOCK 8
#define CSA2_HSI_BLOCKS 2048
#define CSA2_HSI_POOL (CSA2_HSI_BLOCK * CSA2_HSI_BLOCKS)
size_t csa2_hsi_pool_workspace_bytes(int32_t T, int64_t N);
csa2_status csa2_hsi_pool(const float* tile_max, const uint32_t* stats, size_t stats_bytes,
                          const void* q_idx, const float* w_idx, const void* k_idx, const int32_t* q_pos,
                          int32_t ratio, int32_t T, int32_t q_per_seq, int64_t N, int32_t* pool,
                          void* workspace, size_t workspace_bytes, void* hip_stream);

/* ---------------------------------------------------------------- reindex
 * Reindex selection (report sec. 2.3.2): a Reindex layer scores only the
 * entries of the candidate pool (csa2_hsi_pool of the preceding Full layer)
 * with its own indexer query over the shared indexer keys, and keeps the first
 * min(k, pool size) pool entries of the order (I_fp64 descending, index
 * ascending), written ASCENDING into indices[t][0..], -1 padded.  I_fp64 is
 * defined as under csa2_index (the Reindex layer's q_idx, w_idx).
 *
 *  pool     int32 [T][CSA2_HSI_POOL]  ascending entry ids in [0, N), then -1
 *           (as csa2_hsi_pool writes it); the visible set is the pool itself
 *  q_idx    bf16 [T][32][128], w_idx fp32 [T][32]: the Reindex layer's query
 *  k_idx    bf16 [B][N][128]: the shared indexer keys
 *  k        must be CSA2_TOPK;  indices int32 [T][k] out
 *  workspace >= csa2_reindex_workspace_bytes(T, k) (about 4.2 MiB per query,
 *           sized for csa2_reindex_mxfp4's dequantised copy of the pool keys;
 *           this call uses only the pool's scores and their summary)
 *  Runs the scan over each query's pool (key rows read through the pool; no
 *  copy) and a selection kernel within each pool (one block per query,
 *  writing entry ids), both on hip_stream.
 */
size_t csa2_reindex_workspace_bytes(int32_t T, int32_t k);
csa2_status csa2_reindex(const int32_t* pool, const void* q_idx, const float* w_idx, const void* k_idx,
                         int32_t T, int32_t q_per_seq, int64_t N, int32_t k, int32_t* indices,
                         void* workspace, size_t workspace_bytes, void* hip_stream);

/* ---------------------------------------------------------- MXFP4 indexer
 * The indexer with FP4 queries and keys (report sec. 2.4.4: DeepSeek-V4 trains
 * its indexer queries and keys for FP4, in the MXFP4 format).  A 128-channel
 * vector is 64 code bytes (E2M1, element 2i in the low nibble of byte i) and
 * 4 E8M0 scale bytes (scale b covers channels 32b .. 32b + 31):
 *   deq(x)[c] = E2M1(code[c]) * 2^(scale[c / 32] - 127)   (scale 255 invalid).
 * Scores, I_fp64, selection order and outputs are those of the bf16 entry
 * points evaluated on the dequantised values (each exact in bf16).  The key
 * stream is 68 bytes per entry instead of 256.
 *
 * csa2_index_mxfp4    as csa2_index, with
 *     q_codes uint8 [T][32][64], q_scales uint8 [T][32][4],
 *     k_codes uint8 [B][N][64],  k_scales uint8 [B][N][4];
 *     stats >= csa2_index_mxfp4_stats_bytes(T, q_per_seq, N): the summary for
 *     csa2_topk_mxfp4 / csa2_hsi_pool_mxfp4, which also carries the
 *     dequantised queries (those calls take no query argument).  One kernel.
 * csa2_topk_mxfp4     as csa2_topk (stats header written the same way).
 * csa2_hsi_pool_mxfp4 as csa2_hsi_pool.
 * csa2_reindex_mxfp4  as csa2_reindex, with the Reindex layer's FP4 query
 *     (q_codes [T][32][64], q_scales [T][32][4]) and the FP4 keys; workspace
 *     >= csa2_reindex_workspace_bytes(T, k).
 */
size_t csa2_index_mxfp4_stats_bytes(int32_t T, int32_t q_per_seq, int64_t N);
csa2_status csa2_index_mxfp4(const uint8_t* q_codes, const uint8_t* q_scales, const float* w_idx,
                             const uint8_t* k_codes, const uint8_t* k_scales, const int32_t* q_pos,
                             int32_t ratio, int32_t T, int32_t q_per_seq, int64_t N, float* scores,
                             float* tile_max, uint32_t* stats, size_t stats_bytes, void* hip_stream);
csa2_status csa2_topk_mxfp4(const float* scores, const float* tile_max, uint32_t* stats, size_t stats_bytes,
                            const float* w_idx, const uint8_t* k_codes, const uint8_t* k_scales,
                            const int32_t* q_pos, int32_t ratio, int32_t T, int32_t q_per_seq, int64_t N,
                            int32_t k, int32_t* indices, void* workspace, size_t workspace_bytes,
                            void* hip_stream);
csa2_status csa2_topk_mxfp4_ex(const float* scores, const float* tile_max, uint32_t* stats, size_t stats_bytes,
                               const float* w_idx, const uint8_t* k_codes, const uint8_t* k_scales,
                               const int32_t* q_pos, int32_t ratio, int32_t T, int32_t q_per_seq, int64_t N,
                               int32_t k, int32_t select, int32_t* indices, void* workspace, size_t workspace_bytes,
                               void* hip_stream);
csa2_status csa2_hsi_pool_mxfp4(const float* tile_max, const uint32_t* stats, size_t stats_bytes,
                                const float* w_idx, const uint8_t* k_codes, const uint8_t* k_scales,
                                const int32_t* q_pos, int32_t ratio, int32_t T, int32_t q_per_seq, int64_t N,
                                int32_t* pool, void* workspace, size_t workspace_bytes, void* hip_stream);
csa2_status csa2_reindex_mxfp4(const int32_t* pool, const uint8_t* q_codes, const uint8_t* q_scales,
                               const float* w_idx, const uint8_t* k_codes, const uint8_t* k_scales, int32_t T,
                               int32_t q_per_seq, int64_t N, int32_t k, int32_t* indices, void* workspace,
                               size_t workspace_bytes, void* hip_stream);

/* ----------------------------------------------------------------- attend
 * Joint sparse + sliding-window attention over an FP4 main-KV cache.  For
 * query t (sequence b) and head h, over the set E_t of
 *   - main rows x_j = dequant(kv[b][indices[t][j]]) for every j with
 *     indices[t][j] >= 0 (FP4 dequantised before attention, report sec. 2.4.4:
 *     x[c] = E2M1(code[c]) * 2^(scale[c/32] - 127), OCP MX format), and
 *   - window rows swa[b][r] for r in [max(0, swa_end[t] - window), swa_end[t])
 *     (report sec. 3.2.2: a query at position i attends SWA keys
 *     [max(s, i-W+1), i]; the caller's SWA tensor starts at row s),
 * it computes z_j = softmax_scale * (q[t][h] . x_j) and
 *   out[t][h] = sum_j e^{z_j - M} x_j / (sum_j e^{z_j - M} + [sink] e^{sink[h] - M}),
 *   lse[t][h] = M + log(denominator),
 * with key = value = x_j (shared-KV MQA, gzher.com reading sec. 4.1) and one
 * softmax over both sets; the optional sink adds exp(sink[h]) to the
 * denominator only (gzher.com reading sec. 4.3).  Logits and sums are fp32;
 * probabilities enter the value product as bf16.  An empty set gives out = 0,
 * lse = -inf.
 *
 *  q        bf16  [T][64][512]
 *  kv_fp4   uint8 [B][N][256]      E2M1 codes, element 2i in the low nibble of byte i
 *  kv_scale uint8 [B][N][16]       E8M0 scales (255 is invalid)
 *  indices  int32 [T][k]           entry ids in [0, N) or -1; duplicates allowed
 *  swa      bf16  [B][S][512]
 *  swa_end  int32 [T]              in [0, S]
 *  sink     fp32  [64] or NULL
 *  window   1..128;  k == 512;  softmax_scale finite and > 0
 *  out      bf16  [T][64][512] out;  lse fp32 [T][64] out or NULL
 *  workspace >= csa2_attend_workspace_bytes(T, k, window, 1)
 */
size_t csa2_attend_workspace_bytes(int32_t T, int32_t k, int32_t window, int32_t n_layers);
csa2_status csa2_attend_fp4(const void* q, const uint8_t* kv_fp4, const uint8_t* kv_scale,
                            const int32_t* indices, const void* swa, const int32_t* swa_end,
                            const float* sink, float softmax_scale, int32_t T, int32_t q_per_seq,
                            int64_t N, int32_t S, int32_t window, int32_t k, void* out, float* lse,
                            void* workspace, size_t workspace_bytes, void* hip_stream);

/* ------------------------------------------------------------ reuse attend
 * Cross-layer Reuse (report sec. 2.3.1): n_layers Reuse layers attend over
 * the index list and main KV published by the latest Full (or Reindex) layer,
 * each with its own query, window KV and sink; nothing is scored or selected.
 * Layer l's output equals csa2_attend_fp4 called with q[l], swa[l], sink[l]
 * and the shared indices/KV, up to rounding: each query-layer's rows are
 * split over work items whose partial results are merged, and the split is
 * chosen per launch shape (T x n_layers), so the merge can round differently
 * from a single-layer call.  The layers run in one launch; their reads of the
 * shared selected rows after the first come from the L2.
 *
 *  n_layers 1..8
 *  q     bf16 [L][T][64][512];  swa bf16 [L][B][S][512];  sink fp32 [L][64] or NULL
 *  out   bf16 [L][T][64][512];  lse fp32 [L][T][64] or NULL
 *  other arguments as csa2_attend_fp4 (swa_end shared by all layers)
 *  workspace >= csa2_attend_workspace_bytes(T, k, window, n_layers)
 */
csa2_status csa2_reuse_attend(int32_t n_layers, const void* q, const uint8_t* kv_fp4,
                              const uint8_t* kv_scale, const int32_t* indices, const void* swa,
                              const int32_t* swa_end, const float* sink, float softmax_scale,
                              int32_t T, int32_t q_per_seq, int64_t N, int32_t S, int32_t window,
                              int32_t k, void* out, float* lse, void* workspace,
                              size_t workspace_bytes, void* hip_stream);

/* ------------------------------------------------- reuse attend, no workspace
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation):
 * csa2_reuse_attend without the workspace arguments, same arguments
 * otherwise, same kernels and results.  Its split-K partials live in a
 * library-owned device array of CSA2_STATIC_SCRATCH_BYTES per GPU, held until
 * the process ends; the call itself allocates nothing.  Every valid call
 * fits: the split (and its partials) is only used for launches of fewer than
 * 256 query-layers, whose csa2_attend_workspace_bytes is at most 30.3 MiB;
 * the call still returns CSA2_ERR_WORKSPACE, before touching any device, if
 * that size ever exceeded the array.  Every call on a GPU shares that GPU's
 * array: calls that may overlap on one GPU (different streams, threads) race
 * and must be serialised by the caller.  The array needs no clearing between calls.
 * Other errors as csa2_reuse_attend; CSA2_ERR_LAUNCH also when the array's
 * device address cannot be looked up for the stream's device.
 */
#define CSA2_STATIC_SCRATCH_BYTES 34603008  /* 33 MiB: every valid call fits */
csa2_status csa2_reuse_attend_static(int32_t n_layers, const void* q, const uint8_t* kv_fp4,
                                     const uint8_t* kv_scale, const int32_t* indices, const void* swa,
                                     const int32_t* swa_end, const float* sink, float softmax_scale,
                                     int32_t T, int32_t q_per_seq, int64_t N, int32_t S, int32_t window,
                                     int32_t k, void* out, float* lse, void* hip_stream);

/* -------------------------------------------------------- attend, extended
 * csa2_attend_fp4 / csa2_reuse_attend (n_layers as there) with the formats the
 * report deploys and the fused output rotation; opts NULL gives exactly
 * csa2_reuse_attend.
 *
 *  kv_format  CSA2_KV_MXFP4: kv_scales E8M0 [B][N][16] (one per 32 channels);
 *             CSA2_KV_E4M3_16 (report sec. 2.4.4: E2M1 with one E4M3 scale per
 *             16 channels, no global scale; 288 B per entry): kv_scales E4M3
 *             [B][N][32], x[c] = E2M1(code[c]) * E4M3(scale[c / 16]).
 *  swa_format CSA2_SWA_BF16: swa bf16 [L][B][S][512] as before;
 *             CSA2_SWA_FP8 (report sec. 2.4.4 keeps the window KV in FP8; the
 *             V4 layout of 448 FP8 + 64 bf16 channels and 8 scale bytes, 584 B
 *             per row): swa is not read; swa_fp8 E4M3 [L][B][S][448] with
 *             swa_scales E8M0 [L][B][S][8] (scale j for channels 64j..64j+63,
 *             j < 7; byte 7 unused), swa_rope bf16 [L][B][S][64] (channels
 *             448..511).
 *  rope_pos   int32 [T] or NULL: the output's channels 448..511 are rotated
 *             by RoPE at position -rope_pos[t] before the bf16 cast (gzher.com
 *             reading sec. 4.3): pair j = (448 + 2j, 449 + 2j), angle
 *             phi = -pos * rope_base^(-2j/64), (x, y) -> (x cos phi - y sin phi,
 *             x sin phi + y cos phi); rope_base > 1 (e.g. 10000).  lse is not
 *             affected.
 * The window tensors, like swa, start at the replay start; all other
 * arguments, the workspace and the errors are those of csa2_reuse_attend.
 */
#define CSA2_KV_MXFP4 0
#define CSA2_KV_E4M3_16 1
#define CSA2_SWA_BF16 0
#define CSA2_SWA_FP8 1
typedef struct csa2_attend_opts {
    int32_t kv_format;
    int32_t swa_format;
    const uint8_t* swa_fp8;
    const void* swa_rope;
    const uint8_t* swa_scales;
    const int32_t* rope_pos;
    float rope_base;
} csa2_attend_opts;
csa2_status csa2_attend_ex(int32_t n_layers, const void* q, const uint8_t* kv_codes, const uint8_t* kv_scales,
                           const int32_t* indices, const void* swa, const int32_t* swa_end, const float* sink,
                           float softmax_scale, int32_t T, int32_t q_per_seq, int64_t N, int32_t S,
                           int32_t window, int32_t k, const csa2_attend_opts* opts, void* out, float* lse,
                           void* workspace, size_t workspace_bytes, void* hip_stream);

/* -------------------------------------------------------------- KV write
 * The write side of the main-KV cache for n_ent new compressed entries: the
 * CSA2 compressor, the indexer-K projection, RoPE and the cache quantisation.
 * DeepSeek-V4.1-Flash report sec. 2.3: CSA2 pools m tokens into one entry
 * without CSA's overlap between neighbouring entries and without its absolute
 * positional embedding, and obtains indexer K by projecting main-KV entries;
 * sec. 2.4.4: the cache is quantised to FP4 after RoPE.  The pooling form is
 * the gated one of the gzher.com DeepSeek-V4 reading (sec. 4.2, HCA) without
 * its bias: for entry e with tokens t = e*m + j, j < m,
 *   C_t = h_t W_kv^T,  Z_t = h_t W_z^T,
 *   pre[e][c] = sum_j softmax_j(Z_{e*m+j}[c]) C_{e*m+j}[c]   (m = 1: pre = C),
 *   k[e] = pre[e] W_ik^T                         (indexer K, before RoPE),
 *   entry[e] = pre[e] with channels 448..511 rotated at position pos[e]:
 *     pair (448 + 2j, 449 + 2j), phi = pos * rope_base^(-2j/64),
 *     (x, y) -> (x cos phi - y sin phi, x sin phi + y cos phi),
 * and entry[e] is quantised into the cache row:
 *   kv_format CSA2_KV_MXFP4: per 32 channels an E8M0 scale 2^(floor(log2 amax) - 2)
 *     (code clamped to 0..254, 127 for an all-zero block), elements x / scale
 *     to the nearest E2M1 value (ties to the even code, saturating at 6);
 *   kv_format CSA2_KV_E4M3_16: per 16 channels the E4M3 value nearest to
 *     amax / 6 (ties to even, saturating at 448), elements x / scale to E2M1
 *     (all codes 0 when the scale is 0).
 * Indexer K is written as bf16 (k_format 0, nearest even) or as an MXFP4 row
 * (k_format 1: 64 code bytes + 4 E8M0 scales per entry, the same rule).
 * Products and sums are fp32 (projections on bf16 matrix cores); a code may
 * differ from the exact-arithmetic result only where the exact value lies
 * within fp32 rounding of a decision boundary.
 *
 *  h        bf16  [n_ent * m][d]     token hidden states, entry e = rows e*m .. e*m + m - 1
 *  w_kv     bf16  [512][d]           row c = weights of output channel c
 *  w_z      bf16  [512][d]           gate weights; ignored (may be NULL) when m == 1
 *  w_ik     bf16  [128][512]         row o = weights of indexer-K channel o
 *  pos      int32 [n_ent]            RoPE position of each entry
 *  rope_base > 1 and finite
 *  m in {1, 2, 4, 8};  d a positive multiple of 32;  n_ent >= 1
 *  kv_codes uint8 [n_ent][256] out;  kv_scales uint8 [n_ent][16] (MXFP4) or [n_ent][32] (E4M3/16) out
 *  k_out    bf16 [n_ent][128] (k_format 0) or uint8 [n_ent][64] (k_format 1) out
 *  k_scales uint8 [n_ent][4] out (k_format 1; ignored otherwise)
 *  workspace >= csa2_kv_write_workspace_bytes(n_ent, m, d), 16-byte aligned;
 *            its contents on entry do not matter
 * Returns CSA2_ERR_INVALID_ARG for a NULL or misaligned pointer or a bad
 * rope_base, CSA2_ERR_UNSUPPORTED for m, d or a format outside the lists,
 * CSA2_ERR_WORKSPACE for a short workspace.  Outputs may not alias inputs.
 */
#define CSA2_K_BF16 0
#define CSA2_K_MXFP4 1
size_t csa2_kv_write_workspace_bytes(int32_t n_ent, int32_t m, int32_t d);
csa2_status csa2_kv_write(const void* h, const void* w_kv, const void* w_z, const void* w_ik, int32_t d,
                          int32_t n_ent, int32_t m, const int32_t* pos, float rope_base, int32_t kv_format,
                          uint8_t* kv_codes, uint8_t* kv_scales, int32_t k_format, void* k_out,
                          uint8_t* k_scales, void* workspace, size_t workspace_bytes, void* hip_stream);

#ifdef __cplusplus
}
#endif
#endif /* CSA2_H */
