/*
 * CSA2 CPU oracle (fp64).  TEST INFRASTRUCTURE ONLY: used by the tests, the
 * smoke check and the benchmark's CPU-baseline leg, never by the product path.
 * It shares no code with the HIP library.  See csa2_oracle.h for layouts.
 *
 * Every function follows the definition on the pages as plainly as possible:
 * no blocking, no fusion, no reordering beyond the loops written here.
 * Threads (OpenMP) only split independent queries / entry ranges; they do not
 * change any arithmetic.
 */
#include "csa2_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define IDX_HEADS 32
#define IDX_DIM 128
#define HEADS 64
#define DIM 512
#define MX_BLOCK 32

/* Threads the OpenMP loops below will use (1 without OpenMP). */
int32_t csa2o_max_threads(void) {
#ifdef _OPENMP
    return (int32_t)omp_get_max_threads();
#else
    return 1;
#endif
}

/* Set the thread count of the OpenMP loops below (n >= 1); returns the previous one.  The
 * results do not depend on it: threads only split independent queries or score chunks. */
int32_t csa2o_set_threads(int32_t n) {
    int32_t prev = csa2o_max_threads();
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
    return prev;
}

/* ---- formats ------------------------------------------------------------ */

/* bf16 bit pattern -> double (exact). */
static double bf16_to_double(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* OCP MX E2M1: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit.
 * exponent field 0 is subnormal (0 or 0.5); otherwise 2^(E-1) * (1 + M/2).
 * The V4.1 report (sec. 2.4.4) uses E2M1 elements with largest magnitude 6. */
double csa2o_e2m1(uint32_t code) {
    uint32_t s = (code >> 3) & 1u, e = (code >> 1) & 3u, m = code & 1u;
    double mag = (e == 0) ? 0.5 * (double)m : ldexp(1.0 + 0.5 * (double)m, (int)e - 1);
    return s ? -mag : mag;
}

/* OCP MX E8M0 shared scale: 2^(e-127); 0xFF encodes NaN. */
double csa2o_e8m0(uint32_t e) {
    if ((e & 0xFFu) == 0xFFu) return NAN;
    return ldexp(1.0, (int)(e & 0xFFu) - 127);
}

/* V4.1 report sec. 2.4.4: the main KV cache is stored in FP4 after RoPE and
 * dequantised before attention.  x[c] = E2M1(code[c]) * scale[c / 32]. */
void csa2o_dequant_row(const uint8_t* codes, const uint8_t* scales, int32_t dim, double* out) {
    for (int32_t c = 0; c < dim; ++c) {
        uint8_t byte = codes[c / 2];
        uint32_t code = (c % 2 == 0) ? (byte & 0x0Fu) : (byte >> 4);
        out[c] = csa2o_e2m1(code) * csa2o_e8m0(scales[c / MX_BLOCK]);
    }
}

/* OCP 8-bit floating point (OFP8) E4M3: 1 sign bit, 4 exponent bits (bias 7),
 * 3 mantissa bits; exponent field 0 holds subnormals m/8 * 2^-6; S.1111.111
 * is NaN (no infinities), so the largest magnitude is 1.75 * 2^8 = 448. */
double csa2o_e4m3(uint32_t code) {
    double sign = (code & 0x80u) ? -1.0 : 1.0;
    uint32_t e = (code >> 3) & 15u, m = code & 7u;
    if (e == 15u && m == 7u) return NAN;
    if (e == 0u) return sign * ldexp((double)m, -9);
    return sign * ldexp(8.0 + (double)m, (int)e - 10);
}

/* V4.1 report sec. 2.4.4 (the evaluated format it selects for the main KV):
 * E2M1 elements with one E4M3 scale per 16 channels and no global scale.
 * x[c] = E2M1(code[c]) * E4M3(scale[c / 16]). */
void csa2o_dequant_row_e4m3(const uint8_t* codes, const uint8_t* scales, int32_t dim, double* out) {
    for (int32_t c = 0; c < dim; ++c) {
        uint8_t byte = codes[c / 2];
        uint32_t code = (c % 2 == 0) ? (byte & 0x0Fu) : (byte >> 4);
        out[c] = csa2o_e2m1(code) * csa2o_e4m3(scales[c / 16]);
    }
}

/* V4.1 report sec. 2.4.4: the SWA KV stays FP8; the V4 reading (sec. 4.3) keeps
 * the RoPE channels in BF16 and the others in FP8, 448 + 64 channels per entry
 * with 8 scale bytes (584 B).  Reading: channels 0..447 are E4M3 with one E8M0
 * scale per 64 channels (scale bytes 0..6; byte 7 unused), channels 448..511
 * bf16. */
void csa2o_dequant_swa_fp8_row(const uint8_t* fp8, const uint16_t* rope, const uint8_t* scales, double* out) {
    for (int c = 0; c < 448; ++c) out[c] = csa2o_e4m3(fp8[c]) * csa2o_e8m0(scales[c / 64]);
    for (int c = 448; c < DIM; ++c) out[c] = bf16_to_double(rope[c - 448]);
}

/* ---- visibility ---------------------------------------------------------- */

/* V4 reading sec. 4.3: the compressed branch sees a compressed block only once
 * every token in it has been seen; V4.1 report sec. 2.3.2 scores exactly the
 * entries the query may see causally.  With ratio m, entry j holds tokens
 * [m*j, m*j + m). */
int64_t csa2o_n_visible(int64_t pos, int32_t ratio, int64_t N) {
    int64_t n = 0;
    while (n < N && (int64_t)ratio * (n + 1) <= pos + 1) ++n; /* plain count */
    return n;
}

/* ---- indexer ------------------------------------------------------------- */

/* V4 reading sec. 4.1 (lightning indexer): I_{t,s} = sum_h w_{t,h} ReLU(q_{t,h} . K_s);
 * V4.1 report sec. 2.3 keeps CSA's indexer form, with 32 heads x 128
 * (sec. 4.2.1).  fp64, channels in order, heads in order, each step one fma. */
double csa2o_index_score(const uint16_t* q, const float* w, const uint16_t* key) {
    double score = 0.0;
    for (int h = 0; h < IDX_HEADS; ++h) {
        double dot = 0.0;
        for (int c = 0; c < IDX_DIM; ++c)
            dot = fma(bf16_to_double(q[h * IDX_DIM + c]), bf16_to_double(key[c]), dot);
        double relu = dot > 0.0 ? dot : 0.0;
        score = fma((double)w[h], relu, score);
    }
    return score;
}

void csa2o_index(const uint16_t* q_idx, const float* w_idx, const uint16_t* k_idx,
                 const int32_t* q_pos, int32_t ratio, int32_t T, int32_t q_per_seq, int64_t N,
                 double* scores) {
    const int64_t chunk = 4096;
    const int64_t nchunks = (N + chunk - 1) / chunk;
    int64_t* n_vis = (int64_t*)malloc((size_t)(T > 0 ? T : 1) * sizeof(int64_t));
    for (int32_t t = 0; t < T; ++t) n_vis[t] = q_pos ? csa2o_n_visible(q_pos[t], ratio, N) : N;
#pragma omp parallel for schedule(dynamic, 1) collapse(2)
    for (int32_t t = 0; t < T; ++t) {
        for (int64_t ch = 0; ch < nchunks; ++ch) {
            int64_t b = t / q_per_seq;
            const uint16_t* q = q_idx + (int64_t)t * IDX_HEADS * IDX_DIM;
            const float* w = w_idx + (int64_t)t * IDX_HEADS;
            int64_t s_end = (ch + 1) * chunk < N ? (ch + 1) * chunk : N;
            for (int64_t s = ch * chunk; s < s_end; ++s) {
                double v = -INFINITY;
                if (s < n_vis[t]) v = csa2o_index_score(q, w, k_idx + (b * N + s) * IDX_DIM);
                scores[(int64_t)t * N + s] = v;
            }
        }
    }
    free(n_vis);
}

/* V4.1 report sec. 2.4.4: DeepSeek-V4 trains its indexer queries and keys for
 * FP4, in the MXFP4 format.  The score is the lightning-indexer score above,
 * evaluated on the dequantised vectors (csa2o_dequant_row, 128 channels, one
 * scale per 32) in the same fp64 operation order. */
double csa2o_index_score_deq(const double* q, const float* w, const double* key) {
    double score = 0.0;
    for (int h = 0; h < IDX_HEADS; ++h) {
        double dot = 0.0;
        for (int c = 0; c < IDX_DIM; ++c) dot = fma(q[h * IDX_DIM + c], key[c], dot);
        double relu = dot > 0.0 ? dot : 0.0;
        score = fma((double)w[h], relu, score);
    }
    return score;
}

void csa2o_index_mx(const uint8_t* q_codes, const uint8_t* q_scales, const float* w_idx,
                    const uint8_t* k_codes, const uint8_t* k_scales, const int32_t* q_pos, int32_t ratio,
                    int32_t T, int32_t q_per_seq, int64_t N, double* scores) {
    const int64_t row_bytes = IDX_DIM / 2, row_scales = IDX_DIM / MX_BLOCK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t t = 0; t < T; ++t) {
        double q[IDX_HEADS * IDX_DIM], key[IDX_DIM];
        for (int h = 0; h < IDX_HEADS; ++h)
            csa2o_dequant_row(q_codes + ((int64_t)t * IDX_HEADS + h) * row_bytes,
                              q_scales + ((int64_t)t * IDX_HEADS + h) * row_scales, IDX_DIM, q + h * IDX_DIM);
        int64_t n_vis = q_pos ? csa2o_n_visible(q_pos[t], ratio, N) : N;
        int64_t b = t / q_per_seq;
        for (int64_t s = 0; s < N; ++s) {
            double v = -INFINITY;
            if (s < n_vis) {
                csa2o_dequant_row(k_codes + (b * N + s) * row_bytes, k_scales + (b * N + s) * row_scales, IDX_DIM, key);
                v = csa2o_index_score_deq(q, w_idx + (int64_t)t * IDX_HEADS, key);
            }
            scores[(int64_t)t * N + s] = v;
        }
    }
}

/* ---- top-k --------------------------------------------------------------- */

typedef struct {
    double score;
    int64_t idx;
} scored_t;

/* Order used for selection: higher score first, lower index on equal scores. */
static int cmp_score_desc_idx_asc(const void* a, const void* b) {
    const scored_t* x = (const scored_t*)a;
    const scored_t* y = (const scored_t*)b;
    if (x->score > y->score) return -1;
    if (x->score < y->score) return 1;
    return (x->idx < y->idx) ? -1 : (x->idx > y->idx);
}

static int cmp_i32(const void* a, const void* b) {
    int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
    return (x > y) - (x < y);
}

/* V4.1 report sec. 2.3: per query the indexer keeps the K best-scoring
 * entries; K = 512 (sec. 4.2.1).  Full sort, keep the first min(k, n). */
int32_t csa2o_topk_row(const double* scores, int64_t n_vis, int32_t k, int32_t* out) {
    scored_t* all = (scored_t*)malloc((size_t)(n_vis > 0 ? n_vis : 1) * sizeof(scored_t));
    for (int64_t s = 0; s < n_vis; ++s) {
        all[s].score = scores[s];
        all[s].idx = s;
    }
    qsort(all, (size_t)n_vis, sizeof(scored_t), cmp_score_desc_idx_asc);
    int32_t n_sel = (int64_t)k < n_vis ? k : (int32_t)n_vis;
    for (int32_t j = 0; j < n_sel; ++j) out[j] = (int32_t)all[j].idx;
    qsort(out, (size_t)n_sel, sizeof(int32_t), cmp_i32);
    for (int32_t j = n_sel; j < k; ++j) out[j] = -1;
    free(all);
    return n_sel;
}

void csa2o_topk(const double* scores, const int32_t* q_pos, int32_t ratio, int32_t T,
                int64_t N, int32_t k, int32_t* indices) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t t = 0; t < T; ++t) {
        int64_t n_vis = q_pos ? csa2o_n_visible(q_pos[t], ratio, N) : N;
        csa2o_topk_row(scores + (int64_t)t * N, n_vis, k, indices + (int64_t)t * k);
    }
}

/* gzher.com reading of DeepSeek-V4, FP4 QAT section: the index scores are
 * quantised from FP32 to BF16 before the top-k selector.  Reading: the exact
 * score rounded to the nearest bf16 value (8 significant bits, ties to the
 * even significand; below 2^-126 a fixed quantum of 2^-133; beyond the largest
 * bf16 value, infinity), returned as a double. */
double csa2o_bf16_round(double x) {
    if (x == 0.0 || !isfinite(x)) return x;
    int e;
    double f = frexp(x, &e);                 /* x = f * 2^e, 0.5 <= |f| < 1 */
    if (e - 1 < -126) return ldexp(rint(ldexp(x, 133)), -133);
    double r = ldexp(rint(ldexp(f, 8)), e - 8);
    if (fabs(r) > 0x1.FEp127) return copysign(INFINITY, r);
    return r;
}

/* Top-k on bf16-rounded scores: every score rounded (csa2o_bf16_round), then
 * csa2o_topk's order (value descending, index ascending). */
void csa2o_topk_bf16(const double* scores, const int32_t* q_pos, int32_t ratio, int32_t T,
                     int64_t N, int32_t k, int32_t* indices) {
    double* r = (double*)malloc((size_t)T * (size_t)N * sizeof(double));
    for (int64_t i = 0; i < (int64_t)T * N; ++i) r[i] = csa2o_bf16_round(scores[i]);
    csa2o_topk(r, q_pos, ratio, T, N, k, indices);
    free(r);
}

/* ---- hierarchical sparse indexer (candidate pool) and Reindex -------------- */

/* DeepSeek-V4.1-Flash report sec. 2.3.2: the first Full layer also selects
 * blocks; each block gets the maximum index score among its positions, the
 * highest-scoring blocks are kept, and the positions they cover form the
 * candidate pool (sec. 4.2.1: at most 2048 blocks of 8 positions, 16384
 * candidates).  Readings: blocks are the aligned runs [block*b, block*b+block)
 * of compressed entries; only visible entries count toward a block's score and
 * its share of the pool; ties between block scores go to the lower block;
 * the pool is written ascending and padded with -1.  Returns the pool size. */
int32_t csa2o_hsi_pool_row(const double* scores, int64_t n_vis, int32_t block, int32_t n_blocks, int32_t* pool) {
    int64_t nb = (n_vis + block - 1) / block;
    scored_t* blk = (scored_t*)malloc((size_t)(nb > 0 ? nb : 1) * sizeof(scored_t));
    for (int64_t b = 0; b < nb; ++b) {
        double m = -INFINITY;
        for (int64_t e = b * block; e < (b + 1) * block && e < n_vis; ++e)
            if (scores[e] > m) m = scores[e];
        blk[b].score = m;
        blk[b].idx = b;
    }
    qsort(blk, (size_t)nb, sizeof(scored_t), cmp_score_desc_idx_asc);
    int64_t n_sel = nb < n_blocks ? nb : n_blocks;
    int32_t* sel = (int32_t*)malloc((size_t)(n_sel > 0 ? n_sel : 1) * sizeof(int32_t));
    for (int64_t j = 0; j < n_sel; ++j) sel[j] = (int32_t)blk[j].idx;
    qsort(sel, (size_t)n_sel, sizeof(int32_t), cmp_i32);
    int32_t cnt = 0;
    for (int64_t j = 0; j < n_sel; ++j)
        for (int64_t e = (int64_t)sel[j] * block; e < ((int64_t)sel[j] + 1) * block && e < n_vis; ++e) pool[cnt++] = (int32_t)e;
    for (int64_t j = cnt; j < (int64_t)n_blocks * block; ++j) pool[j] = -1;
    free(sel);
    free(blk);
    return cnt;
}

void csa2o_hsi_pool(const double* scores, const int32_t* q_pos, int32_t ratio, int32_t T, int64_t N,
                    int32_t block, int32_t n_blocks, int32_t* pool) {
    const int64_t P = (int64_t)n_blocks * block;
#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t t = 0; t < T; ++t) {
        int64_t n_vis = q_pos ? csa2o_n_visible(q_pos[t], ratio, N) : N;
        csa2o_hsi_pool_row(scores + (int64_t)t * N, n_vis, block, n_blocks, pool + (int64_t)t * P);
    }
}

/* Report sec. 2.3.2: a Reindex layer scores only the pool positions of its
 * query (with its own indexer query, over the shared keys, sec. 2.3) and
 * selects its own top-k within the pool, by (score desc, index asc), written
 * ascending and padded with -1.  scores: the Reindex layer's scores of all
 * entries of the row (only pool entries are read). */
void csa2o_reindex_topk(const double* scores, const int32_t* pool, int32_t T, int64_t N, int64_t P, int32_t k,
                        int32_t* out) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t t = 0; t < T; ++t) {
        const int32_t* pl = pool + (int64_t)t * P;
        const double* row = scores + (int64_t)t * N;
        scored_t* cand = (scored_t*)malloc((size_t)(P > 0 ? P : 1) * sizeof(scored_t));
        int64_t n = 0;
        for (int64_t j = 0; j < P; ++j)
            if (pl[j] >= 0) {
                cand[n].score = row[pl[j]];
                cand[n].idx = pl[j];
                ++n;
            }
        qsort(cand, (size_t)n, sizeof(scored_t), cmp_score_desc_idx_asc);
        int32_t n_sel = (int64_t)k < n ? k : (int32_t)n;
        int32_t* o = out + (int64_t)t * k;
        for (int32_t j = 0; j < n_sel; ++j) o[j] = (int32_t)cand[j].idx;
        qsort(o, (size_t)n_sel, sizeof(int32_t), cmp_i32);
        for (int32_t j = n_sel; j < k; ++j) o[j] = -1;
        free(cand);
    }
}

/* ---- attention ----------------------------------------------------------- */

/* V4 reading sec. 4.3: RoPE on the last 64 channels of q, KV entries and the
 * core-attention output, the output rotated at position -i so that it carries
 * relative positions.  Reading: pairs (448 + 2j, 449 + 2j), angle
 * p * base^(-2j/64) for position p; rotation (x, y) -> (x cos - y sin,
 * x sin + y cos). */
void csa2o_rope_rotate(double* v, double pos, double base) {
    for (int j = 0; j < 32; ++j) {
        double theta = pow(base, -2.0 * j / 64.0);
        double phi = pos * theta;
        double x = v[448 + 2 * j], y = v[449 + 2 * j];
        v[448 + 2 * j] = x * cos(phi) - y * sin(phi);
        v[449 + 2 * j] = x * sin(phi) + y * cos(phi);
    }
}

/* V4 reading sec. 4.1: shared-KV MQA, the selected compressed entry is both
 * key and value; sec. 4.3: an SWA branch of the 128 most recent tokens and an
 * optional per-head sink exp(z'_h) in the softmax denominator.  V4.1 report
 * sec. 2.3: each query attends to the selected entries together with the
 * layer-local SWA KV; sec. 3.2.2: window [max(s, i-W+1), i].
 * One softmax over the union (the neshdevtech reading, sec. 3.3.1/3.3.2,
 * concatenates SWA and selected main KV into a single readout).
 * kv_format 0: MXFP4 rows (E8M0 per 32, scales [B][N][16]); 1: E2M1 with E4M3
 * per 16 (scales [B][N][32]).  swa_format 0: bf16 rows [B][S][512]; 1: FP8 rows
 * (swa_fp8 [B][S][448], swa_rope [B][S][64], swa_scales [B][S][8]).  With
 * rope_pos, each output row is rotated at -rope_pos[t] (csa2o_rope_rotate). */
void csa2o_attend_ex(const uint16_t* q, const uint8_t* kv_codes, const uint8_t* kv_scales, int32_t kv_format,
                     const int32_t* indices, const uint16_t* swa, const uint8_t* swa_fp8, const uint16_t* swa_rope,
                     const uint8_t* swa_scales, int32_t swa_format, const int32_t* swa_end, const double* sink,
                     double softmax_scale, int32_t T, int32_t q_per_seq, int64_t N, int32_t S, int32_t window,
                     int32_t k, const int32_t* rope_pos, double rope_base, double* out, double* lse) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t t = 0; t < T; ++t) {
        int64_t b = t / q_per_seq;
        /* gather the rows of this query's attention set: selected entries in
         * the order of the index list, then the window rows in order */
        int32_t n_main = 0;
        for (int32_t j = 0; j < k; ++j)
            if (indices[(int64_t)t * k + j] >= 0) ++n_main;
        int32_t end = swa_end[t];
        int32_t start = end - window > 0 ? end - window : 0;
        int32_t n_swa = end - start;
        int32_t n_rows = n_main + n_swa;
        double* rows = (double*)malloc((size_t)(n_rows > 0 ? n_rows : 1) * DIM * sizeof(double));
        int32_t r = 0;
        for (int32_t j = 0; j < k; ++j) {
            int64_t s = indices[(int64_t)t * k + j];
            if (s < 0) continue;
            if (kv_format == 0)
                csa2o_dequant_row(kv_codes + (b * N + s) * (DIM / 2), kv_scales + (b * N + s) * (DIM / MX_BLOCK),
                                  DIM, rows + (int64_t)r * DIM);
            else
                csa2o_dequant_row_e4m3(kv_codes + (b * N + s) * (DIM / 2), kv_scales + (b * N + s) * (DIM / 16),
                                       DIM, rows + (int64_t)r * DIM);
            ++r;
        }
        for (int32_t i = start; i < end; ++i, ++r) {
            if (swa_format == 0) {
                for (int c = 0; c < DIM; ++c) rows[(int64_t)r * DIM + c] = bf16_to_double(swa[(b * S + i) * DIM + c]);
            } else {
                csa2o_dequant_swa_fp8_row(swa_fp8 + (b * S + i) * 448, swa_rope + (b * S + i) * 64,
                                          swa_scales + (b * S + i) * 8, rows + (int64_t)r * DIM);
            }
        }

        double* z = (double*)malloc((size_t)(n_rows > 0 ? n_rows : 1) * sizeof(double));
        for (int h = 0; h < HEADS; ++h) {
            const uint16_t* qh = q + ((int64_t)t * HEADS + h) * DIM;
            double m = -INFINITY;
            for (int32_t j = 0; j < n_rows; ++j) {
                double dot = 0.0;
                for (int c = 0; c < DIM; ++c) dot += bf16_to_double(qh[c]) * rows[(int64_t)j * DIM + c];
                z[j] = softmax_scale * dot;
                if (z[j] > m) m = z[j];
            }
            if (sink && sink[h] > m) m = sink[h];
            double* o = out + ((int64_t)t * HEADS + h) * DIM;
            for (int c = 0; c < DIM; ++c) o[c] = 0.0;
            double den = 0.0;
            if (m == -INFINITY) { /* nothing to attend to */
                if (lse) lse[(int64_t)t * HEADS + h] = -INFINITY;
                continue;
            }
            for (int32_t j = 0; j < n_rows; ++j) {
                double p = exp(z[j] - m);
                den += p;
                for (int c = 0; c < DIM; ++c) o[c] += p * rows[(int64_t)j * DIM + c];
            }
            if (sink) den += exp(sink[h] - m);
            for (int c = 0; c < DIM; ++c) o[c] /= den;
            if (rope_pos) csa2o_rope_rotate(o, -(double)rope_pos[t], rope_base);
            if (lse) lse[(int64_t)t * HEADS + h] = m + log(den);
        }
        free(z);
        free(rows);
    }
}

void csa2o_attend(const uint16_t* q, const uint8_t* kv_codes, const uint8_t* kv_scales,
                  const int32_t* indices, const uint16_t* swa, const int32_t* swa_end,
                  const double* sink, double softmax_scale, int32_t T, int32_t q_per_seq,
                  int64_t N, int32_t S, int32_t window, int32_t k, double* out, double* lse) {
    csa2o_attend_ex(q, kv_codes, kv_scales, 0, indices, swa, NULL, NULL, NULL, 0, swa_end, sink, softmax_scale, T,
                    q_per_seq, N, S, window, k, NULL, 0.0, out, lse);
}

/* ---- KV write path ------------------------------------------------------- */

/* OCP MX (v1.0) conversion of one value already divided by its block scale to
 * E2M1: round to the nearest of {0, 0.5, 1, 1.5, 2, 3, 4, 6}, ties to the code
 * with a zero mantissa bit, saturating at 6.  Returns the 4-bit code. */
uint32_t csa2o_e2m1_encode(double v) {
    static const double grid[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    double a = fabs(v);
    uint32_t best = 0;
    for (uint32_t c = 1; c < 8; ++c) {
        double dc = fabs(a - grid[c]), db = fabs(a - grid[best]);
        if (dc < db || (dc == db && (c & 1u) == 0u)) best = c;
    }
    return best | (v < 0.0 ? 8u : 0u);
}

/* OFP8 E4M3 encoding: the nearest finite E4M3 value, ties to the even code,
 * saturating at 448. */
uint32_t csa2o_e4m3_encode(double v) {
    uint32_t best = 0;
    double a = fabs(v);
    for (uint32_t c = 1; c < 0x7F; ++c) {
        double dc = fabs(a - csa2o_e4m3(c)), db = fabs(a - csa2o_e4m3(best));
        if (dc < db || (dc == db && (c & 1u) == 0u)) best = c;
    }
    return best | (v < 0.0 && best != 0 ? 0x80u : 0u);
}

/* MXFP4 block of 32 (OCP MX): shared exponent floor(log2 amax) - 2 (the E2M1
 * maximum exponent), E8M0 code clamped to [0, 254]; an all-zero block gets 127. */
void csa2o_quantize_mx_block(const double* x, uint8_t* codes, uint8_t* scale) {
    double amax = 0.0;
    for (int i = 0; i < 32; ++i) amax = fmax(amax, fabs(x[i]));
    int e = 127;
    if (amax > 0.0) {
        int ex;
        frexp(amax, &ex);               /* amax = f * 2^ex, f in [0.5, 1) */
        e = (ex - 1) - 2 + 127;
        if (e < 0) e = 0;
        if (e > 254) e = 254;
    }
    *scale = (uint8_t)e;
    for (int i = 0; i < 32; i += 2) {
        uint32_t lo = csa2o_e2m1_encode(ldexp(x[i], 127 - e));
        uint32_t hi = csa2o_e2m1_encode(ldexp(x[i + 1], 127 - e));
        codes[i / 2] = (uint8_t)(lo | (hi << 4));
    }
}

/* E2M1 block of 16 with an E4M3 scale (the report's main-KV format, sec. 2.4.4;
 * reading: the scale is the E4M3 value nearest to amax / 6, the elements x /
 * scale rounded to E2M1). */
void csa2o_quantize_e4m3_block(const double* x, uint8_t* codes, uint8_t* scale) {
    double amax = 0.0;
    for (int i = 0; i < 16; ++i) amax = fmax(amax, fabs(x[i]));
    uint32_t sc = csa2o_e4m3_encode(amax / 6.0);
    double s = csa2o_e4m3(sc);
    *scale = (uint8_t)sc;
    for (int i = 0; i < 16; i += 2) {
        uint32_t lo = s > 0.0 ? csa2o_e2m1_encode(x[i] / s) : 0u;
        uint32_t hi = s > 0.0 ? csa2o_e2m1_encode(x[i + 1] / s) : 0u;
        codes[i / 2] = (uint8_t)(lo | (hi << 4));
    }
}

/* V4.1 report sec. 2.3: the CSA2 compressor keeps CSA's gated pooling of m
 * tokens into one main-KV entry without CSA's overlap and absolute positional
 * embedding; the V4 reading (sec. 4.2) gives the pooling: C = H W_kv, Z = H W_z,
 * S = softmax over the m tokens of a block (per channel), entry = sum_j S_j C_j
 * (HCA's form; CSA2 drops its bias B); with m = 1 the entry is C.  Indexer K is
 * a projection of the main-KV entry (sec. 2.3); reading: of the pooled entry
 * before RoPE, K = entry W_ik.  RoPE on the last 64 channels at the entry's
 * position (V4 reading sec. 4.3), then the cache is quantised (sec. 2.4.4,
 * after RoPE).  Every step fp64; sums over k in order.
 * h bf16 [n_ent*m][d]; w_kv, w_z bf16 [d][512] (w_z unused when m = 1);
 * w_ik bf16 [512][128]; pos int32 [n_ent].
 * Outputs: entry fp64 [n_ent][512] (after RoPE, before quantisation), the cache
 * (kv_format 0: MXFP4 codes [n][256] + scales [n][16]; 1: E4M3/16 scales [n][32]),
 * k fp64 [n_ent][128] and k_bf16 (nearest even). */
void csa2o_kv_write(const uint16_t* h, const uint16_t* w_kv, const uint16_t* w_z, const uint16_t* w_ik, int32_t d,
                    int32_t n_ent, int32_t m, const int32_t* pos, double rope_base, int32_t kv_format,
                    double* entry, uint8_t* kv_codes, uint8_t* kv_scales, double* k, uint16_t* k_bf16) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t e = 0; e < n_ent; ++e) {
        double* c = entry + (int64_t)e * DIM;
        double* cj = (double*)malloc((size_t)m * DIM * sizeof(double));
        double* zj = (double*)malloc((size_t)m * DIM * sizeof(double));
        for (int j = 0; j < m; ++j) {
            const uint16_t* hr = h + ((int64_t)e * m + j) * d;
            for (int ch = 0; ch < DIM; ++ch) {
                double acc = 0.0, accz = 0.0;
                for (int32_t kk = 0; kk < d; ++kk) {
                    double hv = bf16_to_double(hr[kk]);
                    acc += hv * bf16_to_double(w_kv[(int64_t)kk * DIM + ch]);
                    if (m > 1) accz += hv * bf16_to_double(w_z[(int64_t)kk * DIM + ch]);
                }
                cj[j * DIM + ch] = acc;
                zj[j * DIM + ch] = accz;
            }
        }
        for (int ch = 0; ch < DIM; ++ch) {
            if (m == 1) { c[ch] = cj[ch]; continue; }
            double zmax = -INFINITY, den = 0.0, num = 0.0;
            for (int j = 0; j < m; ++j) zmax = fmax(zmax, zj[j * DIM + ch]);
            for (int j = 0; j < m; ++j) {
                double p = exp(zj[j * DIM + ch] - zmax);
                den += p;
                num += p * cj[j * DIM + ch];
            }
            c[ch] = num / den;
        }
        for (int o = 0; o < IDX_DIM; ++o) {
            double acc = 0.0;
            for (int ch = 0; ch < DIM; ++ch) acc += c[ch] * bf16_to_double(w_ik[(int64_t)ch * IDX_DIM + o]);
            k[(int64_t)e * IDX_DIM + o] = acc;
            /* nearest bf16, ties to even, taken once from the fp64 sum (a 512-term sum
             * can carry more significant bits than fp32 holds, so no fp32 step in
             * between); the rounded value is a bf16 value, so the float conversion of
             * it is exact and its top 16 bits are the bf16 pattern */
            float f = (float)csa2o_bf16_round(acc);
            uint32_t u;
            memcpy(&u, &f, 4);
            k_bf16[(int64_t)e * IDX_DIM + o] = (uint16_t)(u >> 16);
        }
        csa2o_rope_rotate(c, (double)pos[e], rope_base);
        if (kv_format == 0) {
            for (int b = 0; b < DIM / 32; ++b)
                csa2o_quantize_mx_block(c + 32 * b, kv_codes + (int64_t)e * (DIM / 2) + 16 * b,
                                        kv_scales + (int64_t)e * (DIM / 32) + b);
        } else {
            for (int b = 0; b < DIM / 16; ++b)
                csa2o_quantize_e4m3_block(c + 16 * b, kv_codes + (int64_t)e * (DIM / 2) + 8 * b,
                                          kv_scales + (int64_t)e * (DIM / 16) + b);
        }
        free(cj);
        free(zj);
    }
}
