/*
 * CSA2 CPU oracle: plain, slow, fp64 reference of the CSA2 global-attention
 * hot path (indexer scoring, top-k selection, MXFP4 main-KV dequantisation,
 * joint sparse + sliding-window attention, cross-layer Reuse).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link or
 * call this code; only the tests, the smoke check and the benchmark's CPU
 * baseline leg do.  It shares no code, header, table or constant with the HIP
 * library.
 *
 * Sources (the pages this follows):
 *  - DeepSeek-V4.1-Flash report, sec. 2.3 "Compressed Sparse Attention 2" and
 *    2.3.1 (Full / Reindex / Reuse modes), sec. 2.4.4 "FP4 Main KV Cache",
 *    sec. 3.2.2 "SWA Bounded Replay" (window [max(s, i-W+1), i]), sec. 4.2.1
 *    configuration (32 indexer heads x 128, top-k 512, 64 heads x 512, n_win 128).
 *  - gzher.com reading of DeepSeek-V4, sec. 4.1 "CSA" (lightning-indexer score
 *    I_{t,s} = sum_h w_{t,h} ReLU(q_{t,h} . K_s), shared key = value core
 *    attention) and sec. 4.3 (sliding window branch, attention sink formula).
 *  - OCP Microscaling (MX) format: E2M1 element, E8M0 shared scale per 32.
 *
 * Conventions shared with the library's ABI (data layout only):
 *  - bf16 tensors are passed as uint16 bit patterns, row-major.
 *  - MXFP4 rows: 256 bytes of codes per 512-channel entry, element 2i in the
 *    low nibble of byte i, element 2i+1 in the high nibble; 16 E8M0 scale
 *    bytes per entry, scale j covering channels [32j, 32j+32).
 *  - Query t belongs to sequence t / q_per_seq.
 */
#ifndef CSA2_ORACLE_H
#define CSA2_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Threads the oracle's parallel loops use. */
int32_t csa2o_max_threads(void);
int32_t csa2o_set_threads(int32_t n);

/* Value of one E2M1 code (OCP MX): sign bit 3, magnitudes {0,.5,1,1.5,2,3,4,6}. */
double csa2o_e2m1(uint32_t code);
/* E8M0 scale 2^(e-127); e == 255 (NaN in the spec) returns NaN. */
double csa2o_e8m0(uint32_t e);
/* Dequantise one MXFP4 row of `dim` channels (dim % 32 == 0) into out[dim]. */
void csa2o_dequant_row(const uint8_t* codes, const uint8_t* scales, int32_t dim, double* out);

/* Number of compressed entries causally visible to the token at absolute
 * position `pos` with compression ratio m: entry j (covering tokens
 * [m*j, m*j+m)) is visible iff it is complete, m*(j+1) <= pos+1.
 * Capped at N; a negative position sees nothing.  Functions taking a q_pos
 * array treat NULL as "all N entries visible". */
int64_t csa2o_n_visible(int64_t pos, int32_t ratio, int64_t N);

/* Indexer score of one entry: sum_h w[h] * ReLU(q[h] . key) in fp64, dot
 * products accumulated in channel order with fma, heads in order. */
double csa2o_index_score(const uint16_t* q /*[32][128]*/, const float* w /*[32]*/,
                         const uint16_t* key /*[128]*/);

/* Scores of all entries for T queries: scores[t][s] for s < n_vis(t), -inf
 * beyond.  q_pos may be NULL (all visible). Threads over (t, entry chunk). */
void csa2o_index(const uint16_t* q_idx /*[T][32][128]*/, const float* w_idx /*[T][32]*/,
                 const uint16_t* k_idx /*[B][N][128]*/, const int32_t* q_pos /*[T] or NULL*/,
                 int32_t ratio, int32_t T, int32_t q_per_seq, int64_t N,
                 double* scores /*[T][N]*/);

/* Top-k of one score row: the first min(k, n_vis) entries in the order
 * (score descending, index ascending), written ascending by index into
 * out[k], the rest -1.  Returns the number selected. */
int32_t csa2o_topk_row(const double* scores, int64_t n_vis, int32_t k, int32_t* out);

/* Top-k for T rows of scores[T][N] with per-query visibility. */
void csa2o_topk(const double* scores, const int32_t* q_pos, int32_t ratio, int32_t T,
                int64_t N, int32_t k, int32_t* indices /*[T][k]*/);

/* A double rounded to the nearest bf16 value (ties to even), as a double. */
double csa2o_bf16_round(double x);

/* Top-k of the bf16-rounded scores (csa2o_bf16_round, then csa2o_topk). */
void csa2o_topk_bf16(const double* scores, const int32_t* q_pos, int32_t ratio, int32_t T,
                     int64_t N, int32_t k, int32_t* indices /*[T][k]*/);

/* Joint sparse + sliding-window attention for T queries.
 *  q      bf16 [T][64][512]
 *  kv     MXFP4 codes [B][N][256], scales [B][N][16]
 *  indices [T][k], -1 = empty slot
 *  swa    bf16 [B][S][512]; query t attends SWA rows [max(0, end-W), end),
 *         end = swa_end[t]
 *  sink   [64] or NULL: extra exp(sink_h) term in each head's denominator
 *  out    [T][64][512] fp64; lse [T][64] fp64 or NULL
 * Key = value = the dequantised entry.  One softmax over both sets. */
void csa2o_attend(const uint16_t* q, const uint8_t* kv_codes, const uint8_t* kv_scales,
                  const int32_t* indices, const uint16_t* swa, const int32_t* swa_end,
                  const double* sink, double softmax_scale, int32_t T, int32_t q_per_seq,
                  int64_t N, int32_t S, int32_t window, int32_t k, double* out, double* lse);


/* ---- further formats (report sec. 2.4.4) */
/* OFP8 E4M3 value of a code (bias 7, subnormals, S.1111.111 NaN). */
double csa2o_e4m3(uint32_t code);
/* E2M1 row with one E4M3 scale per 16 channels. */
void csa2o_dequant_row_e4m3(const uint8_t* codes, const uint8_t* scales, int32_t dim, double* out);
/* FP8 window row: 448 E4M3 channels with an E8M0 scale per 64, then 64 bf16 channels. */
void csa2o_dequant_swa_fp8_row(const uint8_t* fp8, const uint16_t* rope, const uint8_t* scales, double* out);

/* ---- MXFP4 indexer (report sec. 2.4.4) */
double csa2o_index_score_deq(const double* q /*[32][128]*/, const float* w, const double* key /*[128]*/);
void csa2o_index_mx(const uint8_t* q_codes, const uint8_t* q_scales, const float* w_idx, const uint8_t* k_codes,
                    const uint8_t* k_scales, const int32_t* q_pos, int32_t ratio, int32_t T, int32_t q_per_seq,
                    int64_t N, double* scores);

/* ---- hierarchical sparse indexer and Reindex (report sec. 2.3.2) */
int32_t csa2o_hsi_pool_row(const double* scores, int64_t n_vis, int32_t block, int32_t n_blocks, int32_t* pool);
void csa2o_hsi_pool(const double* scores, const int32_t* q_pos, int32_t ratio, int32_t T, int64_t N, int32_t block,
                    int32_t n_blocks, int32_t* pool);
void csa2o_reindex_topk(const double* scores, const int32_t* pool, int32_t T, int64_t N, int64_t P, int32_t k,
                        int32_t* out);

/* ---- output rotation and attention with formats (V4 reading sec. 4.3) */
void csa2o_rope_rotate(double* v /*[512]*/, double pos, double base);
void csa2o_attend_ex(const uint16_t* q, const uint8_t* kv_codes, const uint8_t* kv_scales, int32_t kv_format,
                     const int32_t* indices, const uint16_t* swa, const uint8_t* swa_fp8, const uint16_t* swa_rope,
                     const uint8_t* swa_scales, int32_t swa_format, const int32_t* swa_end, const double* sink,
                     double softmax_scale, int32_t T, int32_t q_per_seq, int64_t N, int32_t S, int32_t window,
                     int32_t k, const int32_t* rope_pos, double rope_base, double* out, double* lse);

/* ---- KV write path (report sec. 2.3 compressor, sec. 2.4.4 quantisation) */
uint32_t csa2o_e2m1_encode(double v);
uint32_t csa2o_e4m3_encode(double v);
void csa2o_quantize_mx_block(const double* x /*[32]*/, uint8_t* codes /*[16]*/, uint8_t* scale);
void csa2o_quantize_e4m3_block(const double* x /*[16]*/, uint8_t* codes /*[8]*/, uint8_t* scale);
void csa2o_kv_write(const uint16_t* h, const uint16_t* w_kv, const uint16_t* w_z, const uint16_t* w_ik, int32_t d,
                    int32_t n_ent, int32_t m, const int32_t* pos, double rope_base, int32_t kv_format,
                    double* entry, uint8_t* kv_codes, uint8_t* kv_scales, double* k, uint16_t* k_bf16);

#ifdef __cplusplus
}
#endif
#endif
