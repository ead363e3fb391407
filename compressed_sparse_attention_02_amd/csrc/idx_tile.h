// Indexer score of one 16-key tile on v_mfma_f32_16x16x32_bf16, shared by the
// scan (csa2_index) and the candidate pass of the selection (csa2_topk), so
// that both produce bit-identical fp32 scores for the same key.
//
// Score (lightning indexer of DeepSeek-V4, gzher.com reading sec. 4.1, kept by
// CSA2, report sec. 2.3): I(s) = sum_h w_h * ReLU(q_h . K_s), 32 heads x 128.
//
// Operand layout.  Keys are the B operand: lane l holds key l % 16 of the tile
// and, at MFMA step j (0..3), channels 32j + 8(l/16) .. +8 -- 64 contiguous
// bytes of one key row per lane and load instruction.  The query's two
// 16-head halves are the A operands, read from LDS rows of kQRowPad bf16.
// Accumulator register i of half m holds head 16m + 4(l/16) + i of key l % 16.
#pragma once

#include "csa2_common.h"

namespace csa2 {

constexpr int kTileKeys = 16;          // keys per tile
constexpr int kQRowPad = kIdxDim + 8;  // bf16 per q row in LDS (272 B: spreads rows over banks)

// The four 16-byte pieces of key row `row` that lane (col, g) feeds to the MFMA.
__device__ __forceinline__ void load_key_slices(const uint16_t* __restrict__ kseq, int64_t row, int g,
                                                uint4 (&kv)[4]) {
  const uint16_t* kp = kseq + (size_t)row * kIdxDim + g * 8;
#pragma unroll
  for (int j = 0; j < 4; ++j) kv[j] = *reinterpret_cast<const uint4*>(kp + 32 * j);
}

// Per-lane weights in accumulator order: wr[r] = w[16(r/4) + 4g + r%4].
__device__ __forceinline__ void load_head_weights(const float* __restrict__ w_t, int g, float (&wr)[8]) {
#pragma unroll
  for (int r = 0; r < 8; ++r) wr[r] = w_t[16 * (r >> 2) + 4 * g + (r & 3)];
}

// ReLU of a finite float as one integer maximum on its bits (negative values,
// -0 included, have the sign bit set and become +0).
__device__ __forceinline__ float relu_bits(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// x + (x of lane l ^ 16), and x + (x of lane l ^ 32), with the gfx950 lane
// swaps (v_permlane16_swap / v_permlane32_swap: after swapping a copy of x
// with x, the two registers hold a lane's value and its partner's, so their sum
// is the pairwise sum, the same in both lanes of a pair).
__device__ __forceinline__ float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Maximum over each 16-lane row of scores (finite or -inf, never -0 or NaN),
// in every lane of the row.  The scores go through order-preserving signed
// keys (a float's bits, the magnitude bits flipped when negative), whose
// maximum needs no canonicalisation, so each DPP row move (old value INT_MIN, the
// identity) folds into one v_max_i32_dpp.  Partners i^1, i^2, 7-i within 8, 15-i within 16.
__device__ __forceinline__ int score_key(float x) {
  const int k = __float_as_int(x);
  return k ^ ((k >> 31) & 0x7FFFFFFF);
}
__device__ __forceinline__ float row_max16(float x) {
  int k = score_key(x);
  k = max(k, __builtin_amdgcn_update_dpp(INT_MIN, k, kDppXor1, 0xF, 0xF, false));
  k = max(k, __builtin_amdgcn_update_dpp(INT_MIN, k, kDppXor2, 0xF, 0xF, false));
  k = max(k, __builtin_amdgcn_update_dpp(INT_MIN, k, kDppHalfMirror, 0xF, 0xF, false));
  k = max(k, __builtin_amdgcn_update_dpp(INT_MIN, k, kDppMirror, 0xF, 0xF, false));
  return __int_as_float(k ^ ((k >> 31) & 0x7FFFFFFF));
}

// The score of key l % 16 from the two 16-head accumulator halves (register i
// of half m: head 16m + 4(l/16) + i): ReLU, times the head's weight, summed
// over the lane's 8 heads and then over the four lane groups of the column.
// Returned in every lane of that column.
__device__ __forceinline__ float fold_heads(const floatx4& acc0, const floatx4& acc1, const float (&wr)[8]) {
  float part = 0.f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    part = fmaf(wr[r], relu_bits(acc0[r]), part);
    part = fmaf(wr[4 + r], relu_bits(acc1[r]), part);
  }
  return sum_xor32(sum_xor16(part));
}

// fp32 score of key `col` of the tile, returned in every lane of that column
// (all four lane groups).  sq_t: the query's 32 rows in LDS.
__device__ __forceinline__ float tile_score(const uint16_t* __restrict__ sq_t, const uint4 (&kv)[4],
                                            const float (&wr)[8], int col, int g) {
  floatx4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  const uint16_t* q0 = sq_t + col * kQRowPad + 8 * g;
  const uint16_t* q1 = q0 + 16 * kQRowPad;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const bf16x8 bk = as_bf16x8(kv[j]);
    acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8*>(q0 + 32 * j), bk, acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8*>(q1 + 32 * j), bk, acc1, 0, 0, 0);
  }
  return fold_heads(acc0, acc1, wr);
}

// Stage q[t] (32 x 128 bf16) into LDS rows of kQRowPad: 512 chunks of 16 B.
__device__ __forceinline__ void stage_query(uint16_t* __restrict__ sq_t, const uint16_t* __restrict__ q_t,
                                            int tid, int nthreads) {
  for (int i = tid; i < kIdxHeads * kIdxDim / 8; i += nthreads) {
    const int h = i >> 4, c8 = i & 15;
    *reinterpret_cast<uint4*>(&sq_t[h * kQRowPad + c8 * 8]) =
        *reinterpret_cast<const uint4*>(q_t + h * kIdxDim + c8 * 8);
  }
}

// Row stride (floats) of the tile-maximum array: ceil(N/16) rounded up to 4.
__host__ __device__ __forceinline__ int64_t tile_ld(int64_t N) { return (N + 63) / 64 * 4; }

}  // namespace csa2
