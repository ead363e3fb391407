// KV write path (csa2_kv_write): the CSA2 compressor, the indexer-K
// projection, RoPE and the cache quantisation for n_ent new entries.
//
// DeepSeek-V4.1-Flash report sec. 2.3: CSA2 pools m tokens into one main-KV
// entry without CSA's overlap or absolute positional embedding and projects
// indexer K from the main-KV entry.  Pooling (gzher.com DeepSeek-V4 reading,
// sec. 4.2, HCA's gated form without its bias): C = H W_kv, Z = H W_z, per
// channel a softmax of Z over the entry's m tokens weights C.  RoPE on the last
// 64 channels at the entry's position (reading sec. 4.3); the cache is
// quantised after RoPE (report sec. 2.4.4).
//
// Two kernels, no cross-block synchronisation inside either:
//  projection  C (and Z) on v_mfma_f32_16x16x32_bf16.
//              Many tokens (prefill, kvw_proj_many_kernel): an LDS-tiled GEMM,
//              128 tokens x 128 channels per block, double-buffered k steps.
//              (Measured on 4096 x 5120 x 1024: 128 x 128 tiles with 4 or 8
//              waves, 64 x 128 tiles, and global prefetch 2-4 steps ahead all
//              land within 71-85 us; this layout was the fastest.)
//              Few tokens (decode, kvw_proj_few_kernel): the weight stream
//              (512 x d x 2 B per projection) must be in flight on the whole
//              GPU at once, so the hidden dimension is split: the 4 waves of
//              a block take 4 sub-slices and add them in LDS, and blocks take
//              slices whose sums go to the workspace.
//  kvw_finish_kernel  one block per tile of FT tokens (FT/m whole entries):
//              adds the slice sums in slice order, pools, rotates, quantises
//              the cache rows and computes indexer K from the pooled entries
//              held in LDS.  Every sum has a fixed order: the results do not
//              depend on scheduling.
#include "mxfp4.h"

namespace csa2 {

constexpr int kKvwTok = 16;                     // tokens per MFMA tile
constexpr int kKvwChunk = 64;                   // channels per projection wave
constexpr int kKvwChunks = kDim / kKvwChunk;    // 8
constexpr int kKvwThreads = 256;                // projection block: 4 waves
constexpr int kGemmM = 128, kGemmN = 128, kGemmK = 64;  // many-token projection tile
constexpr int kGemmLd = kGemmK + 8;             // LDS row (bf16): 144 B, rows start on different banks
constexpr int kGemmThreads = 512;               // many-token projection block: 8 waves
constexpr int kKvwFinThreads = 1024;            // finish block
constexpr int kKvwFinMaxTok = 16;               // largest finish tile (many tokens)
constexpr int kKvwFewMaxTok = 8;                // largest finish tile (few tokens)
constexpr int kKvwFewMaxSplit = 8;              // most hidden-dimension slices (few tokens)
constexpr int kKvwMinWaveSlice = 128;           // smallest hidden-dimension slice per wave (few tokens)
constexpr int kKvwWantWaves = 1024;             // projection waves aimed at (few tokens)
constexpr int kKvwManyMin = 1024;               // tokens from which the many-token projection is used

struct KvwPlan {
  int64_t n_tok;
  bool many;
  int tok_tiles;  // 16-token tiles
  int ksplit;     // hidden-dimension slices (blocks along z), 1 for many tokens
  int kper;       // slice length per block (multiple of 128 for few tokens)
  int ft;         // finish tile (tokens): 16 for many tokens, max(4, m) otherwise
  int fin_blocks;
  size_t off_z, total;  // workspace layout (bytes)
};

static size_t kvw_round(size_t b) { return (b + 255) & ~(size_t)255; }

static KvwPlan kvw_plan(int32_t n_ent, int32_t m, int32_t d) {
  KvwPlan p;
  p.n_tok = (int64_t)n_ent * m;
  p.tok_tiles = (int)((p.n_tok + kKvwTok - 1) / kKvwTok);
  p.many = p.n_tok >= kKvwManyMin;
  if (p.many) {
    p.ksplit = 1;
    p.kper = d;
    p.ft = kKvwFinMaxTok;
  } else {
    // blocks along the hidden dimension: ~kKvwWantWaves waves, each at least kKvwMinWaveSlice long
    const int64_t per_split = (int64_t)p.tok_tiles * kKvwChunks * 4;
    int64_t ks = (kKvwWantWaves + per_split - 1) / per_split;
    const int64_t kmax = d / (4 * kKvwMinWaveSlice) > 0 ? d / (4 * kKvwMinWaveSlice) : 1;
    if (ks > kmax) ks = kmax;
    if (ks > kKvwFewMaxSplit) ks = kKvwFewMaxSplit;
    const int q = (d + 127) / 128;  // 128-wide groups
    p.kper = (int)((q + ks - 1) / ks) * 128;
    p.ksplit = (d + p.kper - 1) / p.kper;
    p.ft = m > 4 ? m : 4;
  }
  p.fin_blocks = (int)((p.n_tok + p.ft - 1) / p.ft);
  const size_t part = (size_t)p.ksplit * p.n_tok * kDim * sizeof(float);
  p.off_z = kvw_round(part);
  p.total = p.off_z + (m > 1 ? kvw_round(part) : 0);
  return p;
}

// One 32-wide step of a wave's 16-token tile(s) x 64 channels: A rows from hr
// (token rows of kTT tiles, 16 * d apart), B rows from wr / zr (16-channel
// groups 16 * d apart).
template <int kTT, bool kZ>
__device__ __forceinline__ void proj_steps(const uint16_t* const* hr, const uint16_t* wr, const uint16_t* zr,
                                           size_t g16, int k0, int k1, floatx4 (&acc)[kTT][4],
                                           floatx4 (&accz)[kTT][4]) {
  constexpr int U = kZ ? 2 : (kTT == 1 ? 4 : 2);  // steps per group of loads
  int k = k0;
  for (; k + 32 * U <= k1; k += 32 * U) {
    uint4 a[U][kTT], b[U][4], z[U][kZ ? 4 : 1];
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int t = 0; t < kTT; ++t) a[u][t] = *reinterpret_cast<const uint4*>(hr[t] + k + 32 * u);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        b[u][c] = *reinterpret_cast<const uint4*>(wr + c * g16 + k + 32 * u);
        if constexpr (kZ) z[u][c] = *reinterpret_cast<const uint4*>(zr + c * g16 + k + 32 * u);
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // every load of the group in flight before the first product
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int t = 0; t < kTT; ++t)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          acc[t][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[u][t]), as_bf16x8(b[u][c]), acc[t][c], 0,
                                                              0, 0);
          if constexpr (kZ)
            accz[t][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[u][t]), as_bf16x8(z[u][c]), accz[t][c],
                                                                 0, 0, 0);
        }
  }
  for (; k < k1; k += 32) {
    uint4 a[kTT];
#pragma unroll
    for (int t = 0; t < kTT; ++t) a[t] = *reinterpret_cast<const uint4*>(hr[t] + k);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint4 b = *reinterpret_cast<const uint4*>(wr + c * g16 + k);
#pragma unroll
      for (int t = 0; t < kTT; ++t)
        acc[t][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[t]), as_bf16x8(b), acc[t][c], 0, 0, 0);
      if constexpr (kZ) {
        const uint4 z = *reinterpret_cast<const uint4*>(zr + c * g16 + k);
#pragma unroll
        for (int t = 0; t < kTT; ++t)
          accz[t][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[t]), as_bf16x8(z), accz[t][c], 0, 0, 0);
      }
    }
  }
}

// part[split][token][channel] (and at part + zoff for Z): register i of lane l
// of tile t holds token 16t + 4(l/16) + i and channel l % 16 of each 16-channel group.

// Many tokens: an LDS-tiled GEMM.  Block tile 128 tokens x 128 output channels
// (C channels, then Z channels for m > 1), k in steps of 64 through two LDS
// buffers (the next step's global loads are in flight while the current one is
// multiplied); 8 waves in 2 x 4, each 64 tokens x 32 channels (4 x 2 MFMA
// tiles), both 32-wide halves of a step read from LDS before the products.
// grid (ceil(n_tok / 128), 512 * projections / 128).
template <int PA, int PB>
__device__ __forceinline__ void gemm_gload(uint4 (&ra)[PA], uint4 (&rb)[PB], const uint16_t* const (&ha)[PA],
                                           const uint16_t* const (&wb)[PB], int k, bool in) {
#pragma unroll
  for (int j = 0; j < PA; ++j) ra[j] = in ? *reinterpret_cast<const uint4*>(ha[j] + k) : uint4{0u, 0u, 0u, 0u};
#pragma unroll
  for (int j = 0; j < PB; ++j) rb[j] = in ? *reinterpret_cast<const uint4*>(wb[j] + k) : uint4{0u, 0u, 0u, 0u};
}

template <int PA, int PB>
__device__ __forceinline__ void gemm_lstore(const uint4 (&ra)[PA], const uint4 (&rb)[PB], uint16_t* A, uint16_t* B,
                                            int lr, int lc) {
#pragma unroll
  for (int j = 0; j < PA; ++j) *reinterpret_cast<uint4*>(&A[(lr + (kGemmThreads / 8) * j) * kGemmLd + lc]) = ra[j];
#pragma unroll
  for (int j = 0; j < PB; ++j) *reinterpret_cast<uint4*>(&B[(lr + (kGemmThreads / 8) * j) * kGemmLd + lc]) = rb[j];
}

template <bool kZ>
__global__ __launch_bounds__(kGemmThreads) void kvw_proj_many_kernel(const uint16_t* __restrict__ h,
                                                                     const uint16_t* __restrict__ w_kv,
                                                                     const uint16_t* __restrict__ w_z, int64_t n_tok,
                                                                     int32_t d, float* __restrict__ part, size_t zoff) {
  constexpr int PA = kGemmM * 8 / kGemmThreads, PB = kGemmN * 8 / kGemmThreads;  // 16-byte pieces per thread
  constexpr int TI = 4, TJ = 2;                                                   // MFMA tiles per wave
  __shared__ __align__(16) uint16_t As[2][kGemmM * kGemmLd];
  __shared__ __align__(16) uint16_t Bs[2][kGemmN * kGemmLd];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3, r16 = lane & 15, g = lane >> 4;
  const int64_t m0 = (int64_t)blockIdx.x * kGemmM;
  const int n0 = blockIdx.y * kGemmN;  // 0..1023: C channels, then Z channels
  const uint16_t* W = (kZ && n0 >= kDim) ? w_z : w_kv;
  const int c0 = n0 & (kDim - 1);
  // global -> LDS: thread tid moves 16 B of rows tid / 8 + 64 j, columns 8 (tid % 8) ..
  const int lr = tid >> 3, lc = 8 * (tid & 7);
  const uint16_t* ha_[PA];
  const uint16_t* wb_[PB];
#pragma unroll
  for (int j = 0; j < PA; ++j) {
    const int64_t row = m0 + lr + (kGemmThreads / 8) * j;  // rows past n_tok read the last token; not stored
    ha_[j] = h + (size_t)(row < n_tok ? row : n_tok - 1) * d + lc;
  }
#pragma unroll
  for (int j = 0; j < PB; ++j) wb_[j] = W + (size_t)(c0 + lr + (kGemmThreads / 8) * j) * d + lc;
  const uint16_t* const (&ha)[PA] = ha_;
  const uint16_t* const (&wb)[PB] = wb_;
  uint4 ra[PA], rb[PB];
  floatx4 acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  // d is a multiple of 32: a 16-byte piece is wholly inside or past the end (zeros)
  gemm_gload<PA, PB>(ra, rb, ha, wb, 0, lc < d);
  gemm_lstore<PA, PB>(ra, rb, As[0], Bs[0], lr, lc);
  __syncthreads();
  const int nk = (d + kGemmK - 1) / kGemmK;
  for (int t = 0; t < nk; ++t) {
    const int buf = t & 1;
    if (t + 1 < nk) gemm_gload<PA, PB>(ra, rb, ha, wb, (t + 1) * kGemmK, (t + 1) * kGemmK + lc < d);
    uint4 a0[TI], a1[TI], b0[TJ], b1[TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const uint16_t* row = &As[buf][(64 * wm + 16 * i + r16) * kGemmLd + 8 * g];
      a0[i] = *reinterpret_cast<const uint4*>(row);
      a1[i] = *reinterpret_cast<const uint4*>(row + 32);
    }
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const uint16_t* row = &Bs[buf][(32 * wn + 16 * j + r16) * kGemmLd + 8 * g];
      b0[j] = *reinterpret_cast<const uint4*>(row);
      b1[j] = *reinterpret_cast<const uint4*>(row + 32);
    }
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a0[i]), as_bf16x8(b0[j]), acc[i][j], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a1[i]), as_bf16x8(b1[j]), acc[i][j], 0, 0, 0);
    // the other buffer was last read in step t - 1, before the barrier that ended it
    if (t + 1 < nk) gemm_lstore<PA, PB>(ra, rb, As[buf ^ 1], Bs[buf ^ 1], lr, lc);
    __syncthreads();
  }
  float* out = (kZ && n0 >= kDim) ? part + zoff : part;
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t tk = m0 + 64 * wm + 16 * i + 4 * g + r;
      if (tk < n_tok) {
#pragma unroll
        for (int j = 0; j < TJ; ++j) out[(size_t)tk * kDim + c0 + 32 * wn + 16 * j + r16] = acc[i][j][r];
      }
    }
}

// Few tokens: grid (tok_tiles, 8, ksplit); the block's slice [z * kper, +kper) is
// cut into 4 sub-slices (multiples of 32), one per wave, added in LDS in wave order.
template <bool kZ>
__global__ __launch_bounds__(kKvwThreads) void kvw_proj_few_kernel(const uint16_t* __restrict__ h,
                                                                   const uint16_t* __restrict__ w_kv,
                                                                   const uint16_t* __restrict__ w_z, int64_t n_tok,
                                                                   int32_t d, int kper, float* __restrict__ part,
                                                                   size_t zoff) {
  __shared__ float red[3][kZ ? 2 : 1][16][64];  // waves 1..3: their 16 x 4 x 4 (+ Z) sums by lane
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int64_t tok = (int64_t)blockIdx.x * kKvwTok + r16;
  const int ch0 = blockIdx.y * kKvwChunk + r16;
  const int sub = kper / 4;
  int k0 = blockIdx.z * kper + wave * sub;
  int k1 = k0 + sub;
  if (k1 > d) k1 = d;
  if (k0 > k1) k0 = k1;
  const uint16_t* hr[1] = {h + (size_t)(tok < n_tok ? tok : n_tok - 1) * d + 8 * g};
  const uint16_t* wr = w_kv + (size_t)ch0 * d + 8 * g;
  const uint16_t* zr = kZ ? w_z + (size_t)ch0 * d + 8 * g : nullptr;
  floatx4 acc[1][4], accz[1][4];
#pragma unroll
  for (int c = 0; c < 4; ++c) acc[0][c] = accz[0][c] = floatx4{0.f, 0.f, 0.f, 0.f};
  proj_steps<1, kZ>(hr, wr, zr, (size_t)16 * d, k0, k1, acc, accz);
  if (wave > 0) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        red[wave - 1][0][4 * c + i][lane] = acc[0][c][i];
        if constexpr (kZ) red[wave - 1][kZ ? 1 : 0][4 * c + i][lane] = accz[0][c][i];
      }
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 0; w < 3; ++w)
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[0][c][i] += red[w][0][4 * c + i][lane];
        if constexpr (kZ) accz[0][c][i] += red[w][kZ ? 1 : 0][4 * c + i][lane];
      }
  float* out = part + (size_t)blockIdx.z * n_tok * kDim;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t tk = (int64_t)blockIdx.x * kKvwTok + 4 * g + i;
    if (tk < n_tok) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        out[(size_t)tk * kDim + ch0 + 16 * c] = acc[0][c][i];
        if constexpr (kZ) out[zoff + (size_t)tk * kDim + ch0 + 16 * c] = accz[0][c][i];
      }
    }
  }
}

// ---- quantisation rules (fp32)

// E2M1 code of v (already divided by the block scale): the nearest of
// {0, .5, 1, 1.5, 2, 3, 4, 6}, ties to the even code, saturating at 6; sign in bit 3.
__device__ __forceinline__ uint32_t e2m1_code(float v) {
  const float a = fabsf(v);
  const uint32_t mag = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) + (a >= 3.5f) + (a > 5.0f);
  return mag | (v < 0.f ? 8u : 0u);
}

// Nearest E4M3 code of v >= 0: ties to the even code, saturating at 448 (0x7E).
__device__ __forceinline__ uint32_t e4m3_code_pos(float v) {
  if (!(v > 0.f)) return 0u;
  const float a = fminf(v, 448.f);
  int ex;
  frexpf(a, &ex);
  const int e = ex - 1 > -6 ? ex - 1 : -6;  // binade; below 2^-6 the subnormal step 2^-9
  const float q = ldexpf(a, 3 - e);          // in units of the step 2^(e-3): exact
  float r = floorf(q);
  const float fr = q - r;
  if (fr > 0.5f || (fr == 0.5f && fmodf(r, 2.f) == 1.f)) r += 1.f;
  const int ri = (int)r;  // 0..16; 16 carries into the next binade
  const int code = e > -6 ? (e + 7) * 8 + (ri - 8) : ri;
  return (uint32_t)(code > 0x7E ? 0x7E : code);
}

__device__ __forceinline__ float e4m3_value(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, mm = b & 7u;
  return e == 0 ? (float)mm * 0x1p-9f : __uint_as_float(((e + 120u) << 23) | (mm << 20));
}

// E8M0 code of a block with largest magnitude amax (OCP MX: floor(log2 amax) - 2).
__device__ __forceinline__ uint32_t mx_scale_code(float amax) {
  if (!(amax > 0.f)) return 127u;
  int ex;
  frexpf(amax, &ex);
  const int e = ex - 1 - 2 + 127;
  return (uint32_t)(e < 0 ? 0 : e > 254 ? 254 : e);
}

// max over the 8 lanes of a half row, the 16 lanes of a DPP row, or 32 lanes
__device__ __forceinline__ float max_half_row(float v) {
  v = fmaxf(v, dpp_f32<kDppXor1>(v));
  v = fmaxf(v, dpp_f32<kDppXor2>(v));
  return fmaxf(v, dpp_f32<kDppHalfMirror>(v));
}
__device__ __forceinline__ float max_row(float v) {
  v = max_half_row(v);
  return fmaxf(v, dpp_f32<kDppMirror>(v));
}
__device__ __forceinline__ float max_32(float v) {
  v = max_row(v);
  return fmaxf(v, __shfl_xor(v, 16));
}

// MXFP4 quantisation of 64 values, one per lane (blocks of 32 lanes).  Returns
// the byte of the lane's pair (valid on even lanes) and the block's scale.
__device__ __forceinline__ uint32_t mx_quant_lane(float v, uint32_t* scale) {
  const uint32_t sc = mx_scale_code(max_32(fabsf(v)));
  *scale = sc;
  const uint32_t code = e2m1_code(v * ldexpf(1.f, 127 - (int)sc));
  return code | (dpp_u32<kDppXor1>(code) << 4);
}

// E2M1 with an E4M3 scale per 16 lanes.
__device__ __forceinline__ uint32_t e4m3_quant_lane(float v, uint32_t* scale) {
  const uint32_t sc = e4m3_code_pos(max_row(fabsf(v)) / 6.f);
  *scale = sc;
  const float s = e4m3_value(sc);
  const uint32_t code = s > 0.f ? e2m1_code(v / s) : 0u;
  return code | (dpp_u32<kDppXor1>(code) << 4);
}

// One block per tile of ft tokens (ft / m whole entries).  kFew: ft <= 8 and up
// to kKvwFewMaxSplit slices; otherwise ft <= 16 and one slice.
template <bool kFew>
__global__ __launch_bounds__(kKvwFinThreads) void kvw_finish_kernel(
    const float* __restrict__ part, size_t zoff, int ksplit, int64_t n_tok, int m, int ft,
    const uint16_t* __restrict__ w_ik, const int32_t* __restrict__ pos, double log2_base, int kv_format,
    uint8_t* __restrict__ kv_codes, uint8_t* __restrict__ kv_scales, int k_format, void* __restrict__ k_out,
    uint8_t* __restrict__ k_scales) {
  constexpr int kFt = kFew ? kKvwFewMaxTok : kKvwFinMaxTok;   // largest tile
  constexpr int kS = kFew ? kKvwFewMaxSplit : 1;              // largest slice count
  constexpr int kP = kFt * kDim / kKvwFinThreads;             // (token, channel) pairs per thread
  // slice sums of C and Z; after pooling the same memory holds the K partials [8][kFt][128]
  __shared__ float sc[2][kFt][kDim];
  __shared__ __align__(16) float pre[kFt][kDim];  // pooled entries before RoPE
  const int tid = threadIdx.x, lane = tid & 63;
  const int64_t t0 = (int64_t)blockIdx.x * ft;
  const int valid = n_tok - t0 < ft ? (int)(n_tok - t0) : ft;
  const int n_e = valid / m;  // m divides ft
  const int64_t e0 = (int64_t)blockIdx.x * (ft / m);
  // W_ik row o, channels 64 g .. 64 g + 63 (for the K stage), loaded first
  const int o = tid & (kIdxDim - 1), g = tid >> 7;
  uint4 wq[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) wq[i] = *reinterpret_cast<const uint4*>(w_ik + (size_t)o * kDim + 64 * g + 8 * i);
  // slice sums of pair p = (token p / 512, channel p % 512), slices in order.  Every
  // load is issued before the first add: addresses are clamped into range and the
  // values past the tile or the slice count are dropped.
  {
    const size_t sstride = (size_t)n_tok * kDim;
    const float* pc = part + (size_t)t0 * kDim;
    const int lim = valid * kDim;
    float v[kS][kP], u[kS][kP];
#pragma unroll
    for (int s = 0; s < kS; ++s)
#pragma unroll
      for (int i = 0; i < kP; ++i) {
        const int p = tid + kKvwFinThreads * i < lim ? tid + kKvwFinThreads * i : lim - 1;
        const size_t off = (size_t)(s < ksplit ? s : 0) * sstride + p;
        v[s][i] = pc[off];
        u[s][i] = m > 1 ? pc[zoff + off] : 0.f;
      }
#pragma unroll
    for (int i = 0; i < kP; ++i) {
      const int p = tid + kKvwFinThreads * i;
      float c = v[0][i], z = u[0][i];
#pragma unroll
      for (int s = 1; s < kS; ++s)
        if (s < ksplit) {
          c += v[s][i];
          z += u[s][i];
        }
      if (p < lim) {
        sc[0][p >> 9][p & (kDim - 1)] = c;
        sc[1][p >> 9][p & (kDim - 1)] = z;
      }
    }
  }
  __syncthreads();
  // pooling, RoPE, quantisation: pair p = (entry p / 512, channel p % 512); a wave holds
  // 64 consecutive channels of one entry
#pragma unroll
  for (int i = 0; i < kP; ++i) {
    const int p = tid + kKvwFinThreads * i;
    if (p < n_e * kDim) {  // uniform per wave
      const int el = p >> 9, ch = p & (kDim - 1);
      const int64_t e = e0 + el;
      float v;
      if (m == 1) {
        v = sc[0][el][ch];
      } else {
        float zmax = -INFINITY;
        for (int j = 0; j < m; ++j) zmax = fmaxf(zmax, sc[1][el * m + j][ch]);
        float den = 0.f, num = 0.f;
        for (int j = 0; j < m; ++j) {
          const float w = expf(sc[1][el * m + j][ch] - zmax);
          den += w;
          num += w * sc[0][el * m + j][ch];
        }
        v = num / den;
      }
      pre[el][ch] = v;
      if (ch >= kDim - 64) {
        // channel 448 + 2j + (lane & 1): pair j with partner lane ^ 1
        const int j = (ch - (kDim - 64)) >> 1;
        const double rev = (double)pos[e] * exp2(-log2_base * (j / 32.0)) * 0.15915494309189535;
        const float fr = (float)(rev - rint(rev));
        const float cs = __builtin_amdgcn_cosf(fr), sn = __builtin_amdgcn_sinf(fr);
        const float ov = dpp_f32<kDppXor1>(v);
        v = (lane & 1) ? ov * sn + v * cs : v * cs - ov * sn;
      }
      uint32_t scl;
      const size_t cb = (size_t)e * (kDim / 2) + (ch >> 1);
      if (kv_format == CSA2_KV_MXFP4) {
        const uint32_t byte = mx_quant_lane(v, &scl);
        if (!(lane & 1)) kv_codes[cb] = (uint8_t)byte;
        if (!(lane & 31)) kv_scales[(size_t)e * (kDim / 32) + (ch >> 5)] = (uint8_t)scl;
      } else {
        const uint32_t byte = e4m3_quant_lane(v, &scl);
        if (!(lane & 1)) kv_codes[cb] = (uint8_t)byte;
        if (!(lane & 15)) kv_scales[(size_t)e * (kDim / 16) + (ch >> 4)] = (uint8_t)scl;
      }
    }
  }
  __syncthreads();
  // indexer K: thread (o, g) adds channels 64 g .. +63 for every entry of the tile
  float (*kred)[kFt][kIdxDim] = reinterpret_cast<float (*)[kFt][kIdxDim]>(&sc[0][0][0]);
  static_assert(sizeof(sc) == 8 * kFt * kIdxDim * sizeof(float), "K partials reuse the slice-sum memory");
  for (int el = 0; el < n_e; ++el) {
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float4 x0 = *reinterpret_cast<const float4*>(&pre[el][64 * g + 8 * i]);
      const float4 x1 = *reinterpret_cast<const float4*>(&pre[el][64 * g + 8 * i + 4]);
      a = fmaf(x0.x, bf16lo(wq[i].x), a);
      a = fmaf(x0.y, bf16hi(wq[i].x), a);
      a = fmaf(x0.z, bf16lo(wq[i].y), a);
      a = fmaf(x0.w, bf16hi(wq[i].y), a);
      a = fmaf(x1.x, bf16lo(wq[i].z), a);
      a = fmaf(x1.y, bf16hi(wq[i].z), a);
      a = fmaf(x1.z, bf16lo(wq[i].w), a);
      a = fmaf(x1.w, bf16hi(wq[i].w), a);
    }
    kred[g][el][o] = a;
  }
  __syncthreads();
  // K[e][o] = sum over the 8 channel groups in order; a wave holds 64 outputs of one entry
#pragma unroll
  for (int i = 0; i < (kFt * kIdxDim + kKvwFinThreads - 1) / kKvwFinThreads; ++i) {
    const int q = tid + kKvwFinThreads * i;
    const int el = q >> 7, oo = q & (kIdxDim - 1);
    if (el < n_e) {  // uniform per wave
      float kv = 0.f;
#pragma unroll
      for (int gg = 0; gg < 8; ++gg) kv += kred[gg][el][oo];
      const int64_t e = e0 + el;
      if (k_format == CSA2_K_BF16) {
        reinterpret_cast<uint16_t*>(k_out)[(size_t)e * kIdxDim + oo] = (uint16_t)f32_to_bf16_rne(kv);
      } else {
        uint32_t scl;
        const uint32_t byte = mx_quant_lane(kv, &scl);
        if (!(lane & 1)) reinterpret_cast<uint8_t*>(k_out)[(size_t)e * kMxRowBytes + (oo >> 1)] = (uint8_t)byte;
        if (!(lane & 31)) k_scales[(size_t)e * kMxScales + (oo >> 5)] = (uint8_t)scl;
      }
    }
  }
}

}  // namespace csa2

using namespace csa2;

static bool kvw_shape_ok(int32_t n_ent, int32_t m, int32_t d) {
  return n_ent >= 1 && (m == 1 || m == 2 || m == 4 || m == 8) && d >= 32 && d % 32 == 0 &&
         (int64_t)n_ent * m < ((int64_t)1 << 30);
}

extern "C" size_t csa2_kv_write_workspace_bytes(int32_t n_ent, int32_t m, int32_t d) {
  if (!kvw_shape_ok(n_ent, m, d)) return 0;
  return kvw_plan(n_ent, m, d).total;
}

extern "C" csa2_status csa2_kv_write(const void* h, const void* w_kv, const void* w_z, const void* w_ik, int32_t d,
                                     int32_t n_ent, int32_t m, const int32_t* pos, float rope_base,
                                     int32_t kv_format, uint8_t* kv_codes, uint8_t* kv_scales, int32_t k_format,
                                     void* k_out, uint8_t* k_scales, void* workspace, size_t workspace_bytes,
                                     void* hip_stream) {
  if (!h || !w_kv || !w_ik || !pos || !kv_codes || !kv_scales || !k_out || (m > 1 && !w_z) ||
      (k_format == CSA2_K_MXFP4 && !k_scales))
    return CSA2_ERR_INVALID_ARG;
  if (!aligned16(h) || !aligned16(w_kv) || (m > 1 && !aligned16(w_z)) || !aligned16(w_ik) || !aligned16(pos) ||
      !aligned16(kv_codes) || !aligned16(kv_scales) || !aligned16(k_out) ||
      (k_format == CSA2_K_MXFP4 && !aligned16(k_scales)))
    return CSA2_ERR_INVALID_ARG;
  if (n_ent < 1 || d < 1 || !(rope_base > 1.f) || !(rope_base < INFINITY)) return CSA2_ERR_INVALID_ARG;
  if (!kvw_shape_ok(n_ent, m, d) || (kv_format != CSA2_KV_MXFP4 && kv_format != CSA2_KV_E4M3_16) ||
      (k_format != CSA2_K_BF16 && k_format != CSA2_K_MXFP4))
    return CSA2_ERR_UNSUPPORTED;
  const KvwPlan p = kvw_plan(n_ent, m, d);
  if (!workspace || !aligned16(workspace) || workspace_bytes < p.total) return CSA2_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)hip_stream;
  float* part = (float*)workspace;
  const size_t zoff = p.off_z / sizeof(float);
  const uint16_t *hh = (const uint16_t*)h, *wk = (const uint16_t*)w_kv, *wz = (const uint16_t*)w_z;
  (void)hipGetLastError();
  if (p.many) {
    const dim3 grid((unsigned)((p.n_tok + kGemmM - 1) / kGemmM), (m > 1 ? 2 : 1) * kDim / kGemmN);
    if (m > 1)
      hipLaunchKernelGGL(kvw_proj_many_kernel<true>, grid, dim3(kGemmThreads), 0, st, hh, wk, wz, p.n_tok, d, part,
                         zoff);
    else
      hipLaunchKernelGGL(kvw_proj_many_kernel<false>, grid, dim3(kGemmThreads), 0, st, hh, wk, nullptr, p.n_tok, d,
                         part, zoff);
  } else {
    const dim3 grid(p.tok_tiles, kKvwChunks, p.ksplit);
    if (m > 1)
      hipLaunchKernelGGL(kvw_proj_few_kernel<true>, grid, dim3(kKvwThreads), 0, st, hh, wk, wz, p.n_tok, d, p.kper,
                         part, zoff);
    else
      hipLaunchKernelGGL(kvw_proj_few_kernel<false>, grid, dim3(kKvwThreads), 0, st, hh, wk, nullptr, p.n_tok, d,
                         p.kper, part, zoff);
  }
  auto fin = p.many ? kvw_finish_kernel<false> : kvw_finish_kernel<true>;
  hipLaunchKernelGGL(fin, dim3(p.fin_blocks), dim3(kKvwFinThreads), 0, st, (const float*)part, zoff, p.ksplit,
                     p.n_tok, m, p.ft, (const uint16_t*)w_ik, pos, log2((double)rope_base), kv_format, kv_codes,
                     kv_scales, k_format, k_out, k_scales);
  if (hipGetLastError() != hipSuccess) return CSA2_ERR_LAUNCH;
  return CSA2_OK;
}
