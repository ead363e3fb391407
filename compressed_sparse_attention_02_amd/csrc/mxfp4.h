// MXFP4 operands on gfx950: OCP MX E2M1 elements with one E8M0 scale per 32
// (DeepSeek-V4.1-Flash report sec. 2.4.4: FP4 indexer queries and keys as in
// DeepSeek-V4, the MXFP4 format; the main KV cache uses the same element
// format).  Layout of a 128-channel vector: 64 code bytes, element 2i in the
// low nibble of byte i, and 4 scale bytes, scale b covering channels
// 32b .. 32b + 31.
//
// Also the two sources of indexer-key rows the selection kernels read: bf16
// rows and MXFP4 rows (dequantised to bf16 on the way in; every E2M1 value
// times a power of two is exact in bf16, so the fp64 rescoring sees the exact
// values either way).
#pragma once

#include "idx_tile.h"

namespace csa2 {

typedef int v8i32 __attribute__((ext_vector_type(8)));

constexpr int kMxRowBytes = kIdxDim / 2;  // 64 code bytes per 128-channel row
constexpr int kMxScales = kIdxDim / 32;   // 4 scale bytes per row

// E8M0 scale byte s -> fp32 2^(s-127) (s = 0: the subnormal 2^-127; s = 255 is
// not a valid scale).
__device__ __forceinline__ float e8m0_f32(uint32_t s) { return __uint_as_float(s == 0 ? 0x00400000u : (s << 23)); }

// 8 FP4 codes (one 32-bit word, element 2i in the low nibble of byte i) times
// the block scale 2^(s-127) -> 8 bf16 (4 words, element 2i in the low half).
// v_cvt_scalef32_pk_bf16_fp4 converts the two codes of one byte with an fp32
// scale; every E2M1 value times a power of two is exact in bf16 (at most two
// significant bits).
__device__ __forceinline__ uint4 dequant8(uint32_t codes, uint32_t sbyte) {
  const float sc = e8m0_f32(sbyte);
  uint4 r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 0));
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 1));
  r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 2));
  r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 3));
  return r;
}

// Indexer-key rows as bf16: piece(row, i) = channels 8i .. 8i + 7 of the row;
// slices(row, g, kv) = the MFMA B-operand pieces of lane group g (channels
// 32j + 8g .. + 8, j = 0..3, as load_key_slices).  seq(b, N) moves to sequence b.
struct Bf16Keys {
  const uint16_t* k;
  __device__ __forceinline__ Bf16Keys seq(int64_t b, int64_t N) const { return Bf16Keys{k + (size_t)b * N * kIdxDim}; }
  __device__ __forceinline__ uint4 piece(int64_t row, int i) const {
    return *reinterpret_cast<const uint4*>(k + (size_t)row * kIdxDim + 8 * i);
  }
  __device__ __forceinline__ void slices(int64_t row, int g, uint4 (&kv)[4]) const { load_key_slices(k, row, g, kv); }
};

struct Mx4Keys {
  const uint8_t* codes;   // [N][64]
  const uint8_t* scales;  // [N][4]
  __device__ __forceinline__ Mx4Keys seq(int64_t b, int64_t N) const {
    return Mx4Keys{codes + (size_t)b * N * kMxRowBytes, scales + (size_t)b * N * kMxScales};
  }
  __device__ __forceinline__ uint4 piece(int64_t row, int i) const {
    const uint32_t c = *reinterpret_cast<const uint32_t*>(codes + (size_t)row * kMxRowBytes + 4 * i);
    return dequant8(c, scales[(size_t)row * kMxScales + (i >> 2)]);
  }
  __device__ __forceinline__ void slices(int64_t row, int g, uint4 (&kv)[4]) const {
    const uint32_t s4 = *reinterpret_cast<const uint32_t*>(scales + (size_t)row * kMxScales);
    uint32_t c[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) c[j] = *reinterpret_cast<const uint32_t*>(codes + (size_t)row * kMxRowBytes + 16 * j + 4 * g);
#pragma unroll
    for (int j = 0; j < 4; ++j) kv[j] = dequant8(c[j], (s4 >> (8 * j)) & 255u);
  }
};

// ---- the scan's tile on v_mfma_scale_f32_16x16x128_f8f6f4 (both operands E2M1)
//
// One instruction covers a 16 x 16 x 128 product: lane l supplies row l % 16 of
// A (a head) or column l % 16 of B (a key) for channels 32(l/16) .. + 32, i.e.
// code bytes 16(l/16) .. + 16 of that row, with that block's scale byte; the
// accumulator layout is the bf16 tile's (register i: row 4(l/16) + i, column
// l % 16), so the head fold is shared.

// This lane's A operands of query row q (codes [32][64], scales [32][4]):
// heads l % 16 and 16 + l % 16.
__device__ __forceinline__ void load_query_mx(const uint8_t* __restrict__ qc, const uint8_t* __restrict__ qs, int col,
                                              int g, uint4 (&qa)[2], uint32_t (&qsc)[2]) {
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int h = 16 * m + col;
    qa[m] = *reinterpret_cast<const uint4*>(qc + h * kMxRowBytes + 16 * g);
    qsc[m] = qs[h * kMxScales + g];
  }
}

// This lane's B operand of key row `row`: 16 code bytes and the block's scale.
__device__ __forceinline__ void load_key_mx(const uint8_t* __restrict__ kc, const uint8_t* __restrict__ ks, int64_t row,
                                            int g, uint4* codes, uint32_t* scale) {
  *codes = *reinterpret_cast<const uint4*>(kc + (size_t)row * kMxRowBytes + 16 * g);
  *scale = ks[(size_t)row * kMxScales + g];
}

__device__ __forceinline__ float tile_score_mx(const uint4 (&qa)[2], const uint32_t (&qsc)[2], uint4 kb, uint32_t ksc,
                                               const float (&wr)[8]) {
  const v8i32 b = {(int)kb.x, (int)kb.y, (int)kb.z, (int)kb.w, 0, 0, 0, 0};
  const v8i32 a0 = {(int)qa[0].x, (int)qa[0].y, (int)qa[0].z, (int)qa[0].w, 0, 0, 0, 0};
  const v8i32 a1 = {(int)qa[1].x, (int)qa[1].y, (int)qa[1].z, (int)qa[1].w, 0, 0, 0, 0};
  const floatx4 z = {0.f, 0.f, 0.f, 0.f};
  // format code 4 = E2M1 for both operands
  const floatx4 acc0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a0, b, z, 4, 4, 0, (int)qsc[0], 0, (int)ksc);
  const floatx4 acc1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a1, b, z, 4, 4, 0, (int)qsc[1], 0, (int)ksc);
  return fold_heads(acc0, acc1, wr);
}

// Upper bound of this lane's share of ||K||^2 for the error bound: its block
// holds 32 values of magnitude at most 6 * 2^(s-127).  +inf when the square
// overflows fp32 (the bound then admits every entry, which stays exact).
__device__ __forceinline__ float mx_block_norm2_bound(uint32_t s) {
  const float sc = e8m0_f32(s);
  return 1152.f * sc * sc;
}

// ---- launch plan of the MXFP4 scan and the layout of the summary it leaves
//
// Summary (32-bit words): header [T][4], fp32 group maxima [T][n_groups],
// fp32 partial maxima of the ||K||^2 bound [B * parts], zero words up to a
// 16-byte boundary, then the dequantised queries, bf16 [T][32][128].  The
// scan writes every word.

constexpr int kMxThreads = 256;                 // 4 waves
constexpr int kMxWaves = kMxThreads / 64;
constexpr int kMxTiles = 8;                     // 16-key tiles per wave per iteration (the score store assumes 8)
constexpr int kMxWaveKeys = 16 * kMxTiles;      // 128
constexpr int kMxChunkKeys = kMxWaveKeys * kMxWaves;  // 512 keys per block iteration
constexpr int kMxBlocks = 2048;                 // blocks per launch the grid aims for (measured: 2048-4096 best)
constexpr int kMxGroupsWanted = 4096;

struct MxPlan {
  int qg = 1, groups = 1, B = 1, blocks_x = 1, slots = 1;
  int64_t n_groups = 8;
  int64_t parts() const { return (int64_t)groups * blocks_x; }
};

__host__ __device__ inline int64_t mx_group_count(int64_t blocks_x, int S) {
  return (blocks_x * kMxTiles * S + 3) / 4 * 4;
}

inline bool mx_plan(int32_t T, int32_t q_per_seq, int64_t N, MxPlan* p) {
  if (T < 1 || q_per_seq < 1 || T % q_per_seq != 0 || N < 1 || N >= ((int64_t)1 << 31)) return false;
  p->qg = q_per_seq == 1 ? 1 : q_per_seq == 2 ? 2 : 4;
  p->groups = (q_per_seq + p->qg - 1) / p->qg;
  p->B = T / q_per_seq;
  const int64_t nchunks = (N + kMxChunkKeys - 1) / kMxChunkKeys;
  int64_t want = (kMxBlocks + (int64_t)p->B * p->groups - 1) / ((int64_t)p->B * p->groups);
  if (want > nchunks) want = nchunks;
  if (want < 1) want = 1;
  p->blocks_x = (int)want;
  const int max_slots = p->qg == 1 ? 4 : p->qg == 2 ? 2 : 1;
  int slots = 1;
  while (slots < max_slots && (int64_t)p->blocks_x * kMxTiles * slots < kMxGroupsWanted) slots *= 2;
  p->slots = slots;
  p->n_groups = mx_group_count(p->blocks_x, slots);
  return p->B <= 65535 && p->groups <= 65535;
}

// Summary: the bf16 scan's three parts, then the dequantised queries.
inline size_t mx_qdeq_off(int T, const MxPlan& p) {  // in 32-bit words, 16-byte aligned
  return align_up((size_t)T * CSA2_STATS_WORDS + (size_t)T * p.n_groups + (size_t)p.B * p.parts(), 4);
}
inline size_t mx_stats_words(int T, const MxPlan& p) {
  return mx_qdeq_off(T, p) + (size_t)T * kIdxHeads * kIdxDim / 2;
}

}  // namespace csa2
