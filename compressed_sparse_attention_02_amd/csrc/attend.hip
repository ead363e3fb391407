// Joint sparse + sliding-window attention over the FP4 main-KV cache
// (csa2_attend_fp4) and its cross-layer Reuse form (csa2_reuse_attend).
//
// What is computed (see csa2.h): for query t and head h, one softmax over the
// union of the selected main-KV rows (dequantised MXFP4, report sec. 2.4.4)
// and the window rows (report sec. 3.2.2), with key = value = the row
// (shared-KV MQA, gzher.com reading sec. 4.1) and an optional sink in the
// denominator (gzher.com reading sec. 4.3).  Reuse layers (report sec. 2.3.1)
// attend over the same rows with their own query and window.
//
// Layout of the work.  The rows of one query are processed in chunks of 32
// (16 chunks of selected rows + up to 4 window chunks).  A chunk is gathered
// and dequantised once into LDS in two bf16 copies:
//   X  [32][512]  (row-major, 16-byte row pad)   -> A operand of S^T = X Q^T
//   XT [512][32]  (transposed, 16-byte row pad)  -> A operand of O^T += X^T P^T
// Each of the 4 waves owns 16 heads.  With heads on the N axis of both
// products (v_mfma_f32_16x16x32_bf16), the accumulator of S^T already holds
// P^T in the B-operand layout of the second product (the 32 rows of a chunk
// are stored in XT in the matching permuted order), and the per-head softmax
// statistics live in the same lanes as that head's O^T accumulators, so no
// cross-lane shuffles are needed except the 4-lane row reductions.
// Chunks of one query are split over work items (split-K); partial (max,
// sum, O) are merged by a combine kernel.  The split is chosen per launch
// shape (queries x layers).  Reuse with several layers runs the layers as
// independent query-layers of one launch (each stages its own chunks: the
// selected rows are the same for every layer, so their second and later
// reads hit the L2); layer l's result equals a single-layer call with q[l] up
// to the rounding of the merge.
#include <mutex>

#include "mxfp4.h"

namespace csa2 {

constexpr int kChunk = 32;
constexpr int kXStride = kDim + 8;      // bf16 elements per X row (1040 B)
constexpr int kXTStride = kChunk + 8;   // bf16 elements per XT row (80 B)
constexpr int kMaxSlots = (CSA2_TOPK + kChunk - 1) / kChunk + (CSA2_MAX_WINDOW + kChunk - 1) / kChunk;  // 20
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.f;  // log2 units: O and l rescaled only when the maximum grows by 2^8

struct AttnArgs {
  const uint16_t* q;        // [L][T][64][512]
  const uint8_t* kv_fp4;    // [B][N][256]
  const uint8_t* kv_scale;  // [B][N][16] E8M0 (kv_format 0) or [B][N][32] E4M3 (kv_format 1)
  const int32_t* indices;   // [T][k]
  const uint16_t* swa;      // [L][B][S][512] (swa_format 0)
  const uint8_t* swa_fp8;   // [L][B][S][448] E4M3 (swa_format 1)
  const uint16_t* swa_rope; // [L][B][S][64] bf16, channels 448..511 (swa_format 1)
  const uint8_t* swa_sc;    // [L][B][S][8] E8M0 per 64 channels (swa_format 1)
  const int32_t* rope_pos;  // [T] or null: the output's last 64 channels rotated at -rope_pos[t]
  double rope_log2_base;
  const int32_t* swa_end;   // [T]
  const float* sink;        // [L][64] or null
  float scale_log2;         // softmax_scale * log2(e)
  int T, q_per_seq, B, S, window, k, L;
  int64_t N;
  int n_main, n_swa;        // chunks of selected rows / of window rows
  int cpw;                  // chunks per work item
  int n_items;              // work items per query-layer (partial slots when > 1)
  uint16_t* out;            // [L][T][64][512]
  float* lse;               // [L][T][64] or null
  uint16_t* part_o;         // [L][T][n_items] slots of 64 x 512 bf16 in 16 x 16 tiles (part_tile_off)
  float* part_ml;           // [L][T][n_items][64][2]  (max in log2 units, sum)
};

struct AttnShared {
  alignas(16) uint16_t X[kChunk * kXStride];
  alignas(16) uint16_t XT[kDim * kXTStride];
  int valid[kChunk];
  float rope[32][2];  // (cos, sin) of the output rotation of pair j (final outputs written here)
};

// Head group (16 heads) of this wave and layer of this block: a four-wave
// block covers the four head groups of one query-layer (wave w takes group
// w, blockIdx.z is the layer); one-wave blocks split a work item's heads over
// four blocks (blockIdx.z = 4 * layer + group).
template <int W>
__device__ __forceinline__ int head_group() { return W == 1 ? (int)(blockIdx.z & 3u) : (int)(threadIdx.x >> 6); }
template <int W>
__device__ __forceinline__ int block_layer() { return W == 1 ? (int)(blockIdx.z >> 2) : (int)blockIdx.z; }

// Two fp32 values rounded to nearest-even bf16 and packed, lo in the low half
// (one v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2_rne(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// Split-K partial slot layout: 64 heads x 512 channels as 16 x 16 tiles,
// head group G (heads 16G..16G+15) outermost, then channel tile ct (channels
// 16ct..16ct+15), then head, then channel: a wave's store of one tile (lane
// (r, g): head r, channels 4g..4g+3) is 512 contiguous bytes, and the combine
// reads whole tiles.  Offset (bf16 elements) of head 16G + r, channel 16ct + c.
__device__ __forceinline__ size_t part_tile_off(int G, int ct, int r, int c) {
  return ((size_t)(G * (kDim / 16) + ct) * 16 + r) * 16 + c;
}

// 16-byte LDS operand read (the offsets used are multiples of 16 bytes).
__device__ __forceinline__ bf16x8 lds_read16(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8*>(__builtin_assume_aligned(p, 16));
}

// OCP E4M3 byte -> fp32 (bias 7, exponent field 0 subnormal; S.1111.111, NaN,
// is not a valid scale and decodes to 480 here).
__device__ __forceinline__ float e4m3_f32(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  const float mag = e == 0 ? (float)m * 0x1p-9f : __uint_as_float(((e + 120u) << 23) | (m << 20));
  return (b & 0x80u) ? -mag : mag;
}

// 8 E2M1 codes times an E4M3 scale -> 8 bf16.  The conversion instruction
// applies only the exponent of its scale, so the codes are converted at scale 1
// and multiplied in fp32: an E2M1 value times an E4M3 value has at most 6
// significant bits, exact in fp32 and in bf16, so dropping the low half is exact.
__device__ __forceinline__ uint4 dequant8_e4m3(uint32_t codes, uint32_t sbyte) {
  const float sc = e4m3_f32(sbyte);
  const uint4 u = dequant8(codes, 127u);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
  uint32_t r[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    r[i] = (__float_as_uint(bf16lo(w[i]) * sc) >> 16) | (__float_as_uint(bf16hi(w[i]) * sc) & 0xFFFF0000u);
  return make_uint4(r[0], r[1], r[2], r[3]);
}

// Channels 8d .. 8d + 7 of window row `row` (flat [L][B][S] index) as bf16:
// a bf16 row, or an FP8 row (E4M3 with an E8M0 scale per 64 channels below
// channel 448, bf16 above; the scale is a power of two, so the conversion
// instruction's scaling is exact).
template <int SWF>
__device__ __forceinline__ uint4 window_piece(const AttnArgs& a, size_t row, int d) {
  if (SWF == CSA2_SWA_BF16) return *reinterpret_cast<const uint4*>(a.swa + row * kDim + 8 * d);
  if (d >= 56) return *reinterpret_cast<const uint4*>(a.swa_rope + row * 64 + 8 * (d - 56));
  const uint2 c = *reinterpret_cast<const uint2*>(a.swa_fp8 + row * 448 + 8 * d);
  const float sc = e8m0_f32(a.swa_sc[row * 8 + (d >> 3)]);
  uint4 r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.x, sc, false));
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.x, sc, true));
  r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.y, sc, false));
  r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.y, sc, true));
  return r;
}

// cos and sin of the inverse-RoPE angle -pos * base^(-2j/64) of pair j: the
// angle in revolutions is formed in fp64 (positions up to 2^31 times
// frequencies up to 1) and reduced to [-1/2, 1/2] there, then v_sin_f32 /
// v_cos_f32, which take revolutions, give the fp32 values.
__device__ __forceinline__ void rope_cs(const AttnArgs& a, int t, int j, float* c, float* s) {
  const double rev = -(double)a.rope_pos[t] * exp2(-a.rope_log2_base * (j / 32.0)) * 0.15915494309189535;
  const float fr = (float)(rev - rint(rev));
  *c = __builtin_amdgcn_cosf(fr);
  *s = __builtin_amdgcn_sinf(fr);
}

// XT rows hold 32 bf16 in four 16-byte blocks; block b of row r is stored at
// position (b + r / 8) % 4 so that the transposing writes of one staging step
// (rows 8d + i for the 64 lanes d) spread over the LDS banks.
__device__ __forceinline__ int xt_off(int row, int blk) { return row * kXTStride + 8 * ((blk + (row >> 3)) & 3); }

// Chunk `c` of query t (layer `layer` for window chunks) in LDS: row group g
// (0..3), lane d holds 8 rows x 8 channels, rows {4g..4g+3, 16+4g..16+4g+3}
// (the 8 rows that form XT column group g), channels 8d..8d+7.
__device__ __forceinline__ int group_row(int g, int r) { return r < 4 ? 4 * g + r : 16 + 4 * g + (r - 4); }

// Write row group g (v: bf16 words, okr: row valid) to X and, transposed, to XT.
__device__ __forceinline__ void write_group(AttnShared& sh, int g, int d, const uint32_t (&v)[8][4],
                                            const int (&okr)[8]) {
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int e = group_row(g, r);
    *reinterpret_cast<uint4*>(&sh.X[e * kXStride + 8 * d]) = make_uint4(v[r][0], v[r][1], v[r][2], v[r][3]);
    if (d == 0) sh.valid[e] = okr[r];
  }
  // transposed copy: XT[8d + i][8g + r] = v[r][i] (channel 8d+i of row r of this group)
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t w[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t lo = (v[2 * p][i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
      const uint32_t hi = (v[2 * p + 1][i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
      w[p] = lo | (hi << 16);
    }
    *reinterpret_cast<uint4*>(&sh.XT[xt_off(8 * d + i, g)]) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// Row group g of a selected-row chunk from its codes and scale bytes (rows of
// -1 slots were read from row 0 and are zeroed here).
template <int KVF>
__device__ __forceinline__ void dequant_group(AttnShared& sh, int g, int d, const int32_t* idx, const uint32_t* codes,
                                              const uint32_t* sbyte) {
  uint32_t v[8][4];
  int okr[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    okr[r] = idx[r] >= 0;
    const uint4 o = KVF == CSA2_KV_MXFP4 ? dequant8(codes[r], sbyte[r]) : dequant8_e4m3(codes[r], sbyte[r]);
    v[r][0] = okr[r] ? o.x : 0u; v[r][1] = okr[r] ? o.y : 0u;
    v[r][2] = okr[r] ? o.z : 0u; v[r][3] = okr[r] ? o.w : 0u;
  }
  write_group(sh, g, d, v, okr);
}

// NG row groups g0, g0 + 1, ... staged by one wave, every load of a kind in
// flight together: the indices, then the codes and scales (selected rows), or
// the window rows.
template <int NG, int KVF, int SWF>
__device__ __forceinline__ void stage_groups(const AttnArgs& a, AttnShared& sh, int t, int b, int c, int layer,
                                             int g0) {
  const int d = threadIdx.x & 63;
  if (c < a.n_main) {
    int32_t idx[NG][8];
#pragma unroll
    for (int j = 0; j < NG; ++j)
#pragma unroll
      for (int r = 0; r < 8; ++r) idx[j][r] = a.indices[(size_t)t * a.k + c * kChunk + group_row(g0 + j, r)];
    uint32_t codes[NG][8], sbyte[NG][8];
#pragma unroll
    for (int j = 0; j < NG; ++j)
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const size_t rowid = (size_t)b * a.N + (idx[j][r] >= 0 ? idx[j][r] : 0);
        codes[j][r] = *reinterpret_cast<const uint32_t*>(a.kv_fp4 + rowid * 256 + 4 * d);
        sbyte[j][r] = KVF == CSA2_KV_MXFP4 ? a.kv_scale[rowid * 16 + (d >> 2)] : a.kv_scale[rowid * 32 + (d >> 1)];
      }
#pragma unroll
    for (int j = 0; j < NG; ++j) dequant_group<KVF>(sh, g0 + j, d, idx[j], codes[j], sbyte[j]);
  } else {
    const int we = a.swa_end[t];
    const int ws = we - a.window > 0 ? we - a.window : 0;
    // window rows two groups at a time (32 registers per group)
#pragma unroll
    for (int j0 = 0; j0 < NG; j0 += 2) {
      uint32_t v[2][8][4];
      int okr[2][8];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if (j0 + j >= NG) continue;  // compile-time
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const int row = ws + (c - a.n_main) * kChunk + group_row(g0 + j0 + j, r);
          okr[j][r] = row < we;
          const int rr = okr[j][r] ? row : (we > 0 ? we - 1 : 0);
          const uint4 x = window_piece<SWF>(a, ((size_t)layer * a.B + b) * a.S + rr, d);
          v[j][r][0] = okr[j][r] ? x.x : 0u; v[j][r][1] = okr[j][r] ? x.y : 0u;
          v[j][r][2] = okr[j][r] ? x.z : 0u; v[j][r][3] = okr[j][r] ? x.w : 0u;
        }
      }
#pragma unroll
      for (int j = 0; j < 2; ++j)
        if (j0 + j < NG) write_group(sh, g0 + j0 + j, d, v[j], okr[j]);
    }
  }
}

// Software-pipelined staging of four-wave blocks: wave g requests the raw
// bytes of its row group of the next chunk (and the indices of the one after)
// before the current chunk's products, and converts them into LDS after.
// Selected rows keep each row's code word (v.x) and scale byte (v.y); window
// rows their 16-byte piece (bf16), or for FP8 rows below channel 448 the
// 8 code bytes (v.x, v.y) and the scale byte (v.z).  Bit r of ok: row r valid.
struct RawGroup {
  uint4 v[8];
  uint32_t ok;
};

__device__ __forceinline__ void load_indices(const AttnArgs& a, int t, int c, int g, int32_t (&idx)[8]) {
  if (c < a.n_main) {
#pragma unroll
    for (int r = 0; r < 8; ++r) idx[r] = a.indices[(size_t)t * a.k + c * kChunk + group_row(g, r)];
  }
}

template <int KVF, int SWF>
__device__ __forceinline__ void load_group_raw(const AttnArgs& a, int t, int b, int c, int layer, int g,
                                               const int32_t (&idx)[8], RawGroup& rg) {
  const int d = threadIdx.x & 63;
  uint32_t ok = 0;
  if (c < a.n_main) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      ok |= (idx[r] >= 0 ? 1u : 0u) << r;
      const size_t rowid = (size_t)b * a.N + (idx[r] >= 0 ? idx[r] : 0);
      rg.v[r].x = *reinterpret_cast<const uint32_t*>(a.kv_fp4 + rowid * 256 + 4 * d);
      rg.v[r].y = KVF == CSA2_KV_MXFP4 ? a.kv_scale[rowid * 16 + (d >> 2)] : a.kv_scale[rowid * 32 + (d >> 1)];
    }
  } else {
    const int we = a.swa_end[t];
    const int ws = we - a.window > 0 ? we - a.window : 0;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int row = ws + (c - a.n_main) * kChunk + group_row(g, r);
      ok |= (row < we ? 1u : 0u) << r;
      const size_t rr = ((size_t)layer * a.B + b) * a.S + (row < we ? row : (we > 0 ? we - 1 : 0));
      if (SWF == CSA2_SWA_BF16) {
        rg.v[r] = *reinterpret_cast<const uint4*>(a.swa + rr * kDim + 8 * d);
      } else if (d >= 56) {
        rg.v[r] = *reinterpret_cast<const uint4*>(a.swa_rope + rr * 64 + 8 * (d - 56));
      } else {
        const uint2 cw = *reinterpret_cast<const uint2*>(a.swa_fp8 + rr * 448 + 8 * d);
        rg.v[r] = make_uint4(cw.x, cw.y, a.swa_sc[rr * 8 + (d >> 3)], 0u);
      }
    }
  }
  rg.ok = ok;
}

// Convert wave g's raw row group of chunk c to bf16 and write it to X and XT.
template <int KVF, int SWF>
__device__ __forceinline__ void store_group_raw(const AttnArgs& a, AttnShared& sh, int c, int g, const RawGroup& rg) {
  const int d = threadIdx.x & 63;
  uint32_t v[8][4];
  int okr[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    okr[r] = (rg.ok >> r) & 1u;
    uint4 o;
    if (c < a.n_main) {
      o = KVF == CSA2_KV_MXFP4 ? dequant8(rg.v[r].x, rg.v[r].y) : dequant8_e4m3(rg.v[r].x, rg.v[r].y);
    } else if (SWF == CSA2_SWA_BF16 || d >= 56) {
      o = rg.v[r];
    } else {
      const float sc = e8m0_f32(rg.v[r].z);
      o.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(rg.v[r].x, sc, false));
      o.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(rg.v[r].x, sc, true));
      o.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(rg.v[r].y, sc, false));
      o.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(rg.v[r].y, sc, true));
    }
    v[r][0] = okr[r] ? o.x : 0u; v[r][1] = okr[r] ? o.y : 0u;
    v[r][2] = okr[r] ? o.z : 0u; v[r][3] = okr[r] ? o.w : 0u;
  }
  write_group(sh, g, d, v, okr);
}

// Stage chunk `c` into LDS: wave g of a 4-wave block takes row group g, a
// one-wave block all four.
template <int KVF, int SWF>
__device__ void stage_chunk(const AttnArgs& a, AttnShared& sh, int t, int b, int c, int layer) {
  if (blockDim.x == 64) stage_groups<4, KVF, SWF>(a, sh, t, b, c, layer, 0);
  else stage_groups<1, KVF, SWF>(a, sh, t, b, c, layer, threadIdx.x >> 6);
}

struct HeadState {
  floatx4 o[32];   // O^T: o[mb][i] = O[head][16*mb + 4*g + i]
  float m;         // running max (log2 units)
  float l;         // running sum (this lane's rows only)
};

__device__ __forceinline__ void load_q(const AttnArgs& a, int layer, int t, int hg, bf16x8* qb) {
  const int lane = threadIdx.x & 63;
  const int head = 16 * hg + (lane & 15), g = lane >> 4;
  const uint4* qp = reinterpret_cast<const uint4*>(a.q + (((size_t)layer * a.T + t) * kHeads + head) * kDim + 8 * g);
#pragma unroll
  for (int j = 0; j < 16; ++j) qb[j] = as_bf16x8(qp[4 * j]);  // channels 32j + 8g .. +8
}

__device__ __forceinline__ void state_init(HeadState& st) {
#pragma unroll
  for (int mb = 0; mb < 32; ++mb) st.o[mb] = floatx4{0.f, 0.f, 0.f, 0.f};
  st.m = -INFINITY;
  st.l = 0.f;
}

// Attend the staged chunk with one query (qb) and fold it into st.
__device__ __forceinline__ void attend_chunk(const AttnArgs& a, const AttnShared& sh, const bf16x8* qb,
                                             HeadState& st) {
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15, g = lane >> 4;
  floatx4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const bf16x8 x0 = lds_read16(&sh.X[r16 * kXStride + 32 * j + 8 * g]);
    const bf16x8 x1 = lds_read16(&sh.X[(16 + r16) * kXStride + 32 * j + 8 * g]);
    s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x0, qb[j], s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x1, qb[j], s1, 0, 0, 0);
  }
  // s0[i]: row 4g+i, s1[i]: row 16+4g+i, both for head (lane & 15)
  float z[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    z[i] = sh.valid[4 * g + i] ? s0[i] * a.scale_log2 : -INFINITY;
    z[4 + i] = sh.valid[16 + 4 * g + i] ? s1[i] * a.scale_log2 : -INFINITY;
  }
  float cm = z[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) cm = fmaxf(cm, z[i]);
  cm = fmaxf(cm, __shfl_xor(cm, 16, 64));
  cm = fmaxf(cm, __shfl_xor(cm, 32, 64));
  const float mtrue = fmaxf(st.m, cm);
  if (mtrue == -INFINITY) return;  // nothing valid so far for this head (uniform per head)
  // Lazy rescaling: the reference maximum st.m stays while this chunk's scores
  // exceed it by at most kRescaleSlack (log2 units), so p <= 2^kRescaleSlack,
  // which bf16 and fp32 hold at full relative precision; (m, l, O) stay
  // consistent, since l and O are both taken relative to st.m.
  const bool grow = mtrue > st.m + kRescaleSlack;  // always on the first valid chunk
  const float mn = grow ? mtrue : st.m;
  const float alpha = exp2f(st.m - mn);  // st.m == -inf -> 0; 1 where the reference stays
  uint32_t pb[4];
  float psum = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float p0 = exp2f(z[2 * i] - mn), p1 = exp2f(z[2 * i + 1] - mn);
    psum += p0 + p1;
    pb[i] = pack_bf16x2_rne(p0, p1);
  }
  // a state with nothing folded in yet (every head of the wave) holds zeros: no rescale
  const bool fresh = __ballot(st.m != -INFINITY) == 0ull;
  st.l = st.l * alpha + psum;
  st.m = mn;
  bf16x8 pv;
  __builtin_memcpy(&pv, pb, 16);
  if (!fresh && __ballot(grow) != 0ull) {
#pragma unroll
    for (int mb = 0; mb < 32; ++mb) st.o[mb] *= alpha;
  }
#pragma unroll
  for (int mb = 0; mb < 32; ++mb) {
    const bf16x8 xa = lds_read16(&sh.XT[xt_off(16 * mb + r16, g)]);
    st.o[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, pv, st.o[mb], 0, 0, 0);
  }
}

// Write the final output of one (layer, query) from a complete state (the
// rotation's (cos, sin) pairs already in sh.rope when a.rope_pos is given).
__device__ void write_final(const AttnArgs& a, const AttnShared& sh, const HeadState& st, int layer, int t,
                            int hg) {
  const int lane = threadIdx.x & 63;
  const int head = 16 * hg + (lane & 15), g = lane >> 4;
  float l = st.l;
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  float m = st.m;
  float den = l, f = 1.f;
  if (a.sink) {
    const float sk = a.sink[(size_t)layer * kHeads + head] * kLog2e;
    const float M = fmaxf(m, sk);
    if (M != -INFINITY) {
      f = (m == -INFINITY) ? 0.f : exp2f(m - M);
      den = l * f + exp2f(sk - M);
      m = M;
    }
  }
  const float inv = (m == -INFINITY || den == 0.f) ? 0.f : f / den;
  uint16_t* op = a.out + (((size_t)layer * a.T + t) * kHeads + head) * kDim + 4 * g;
#pragma unroll
  for (int mb = 0; mb < 32; ++mb) {
    float v[4] = {st.o[mb][0] * inv, st.o[mb][1] * inv, st.o[mb][2] * inv, st.o[mb][3] * inv};
    if (mb >= 28 && a.rope_pos) {  // channels 448..511: pairs (v0, v1), (v2, v3)
      const int j0 = 8 * (mb - 28) + 2 * g;
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const float c = sh.rope[j0 + p][0], sn = sh.rope[j0 + p][1];
        const float x = v[2 * p], y = v[2 * p + 1];
        v[2 * p] = x * c - y * sn;
        v[2 * p + 1] = x * sn + y * c;
      }
    }
    const uint32_t w0 = pack_bf16x2_rne(v[0], v[1]);
    const uint32_t w1 = pack_bf16x2_rne(v[2], v[3]);
    *reinterpret_cast<uint2*>(op + 16 * mb) = make_uint2(w0, w1);
  }
  if (a.lse && g == 0)
    a.lse[((size_t)layer * a.T + t) * kHeads + head] = (m == -INFINITY) ? -INFINITY : (m + log2f(den)) * kLn2;
}

__device__ void write_partial(const AttnArgs& a, const HeadState& st, int layer, int t, int slot, int hg) {
  const int lane = threadIdx.x & 63;
  const int head = 16 * hg + (lane & 15), g = lane >> 4;
  float l = st.l;
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  const size_t slot_id = ((size_t)layer * a.T + t) * a.n_items + slot;
  const size_t base = slot_id * kHeads + head;
  uint16_t* op = a.part_o + slot_id * kHeads * kDim + part_tile_off(hg, 0, lane & 15, 4 * g);
  // bf16 partials (the combine accumulates in fp32), one 512-byte tile per
  // store; streaming stores: they are read once, by the combine kernel
#pragma unroll
  for (int mb = 0; mb < 32; ++mb) {
    const uint32_t w0 = pack_bf16x2_rne(st.o[mb][0], st.o[mb][1]);
    const uint32_t w1 = pack_bf16x2_rne(st.o[mb][2], st.o[mb][3]);
    const u32x2 w = {w0, w1};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x2*>(op + 256 * mb));
  }
  if (g == 0) {
    a.part_ml[base * 2 + 0] = st.m;
    a.part_ml[base * 2 + 1] = l;
  }
}

// grid (n_items, T, L) with four-wave blocks, (n_items, T, 4 L) with one-wave
// blocks.  Work item i of query-layer (t, l) covers chunks [i*cpw,
// min((i+1)*cpw, n_main+n_swa)) (selected rows, then the layer's window
// rows); with FINAL (one item per query-layer) it writes the output, else
// partial slot i.  One-wave blocks take one chunk each (the plan makes it
// so): they stage before the query and the running state are live.
#ifndef CSA2_ATTN_WAVES_PER_SIMD
#define CSA2_ATTN_WAVES_PER_SIMD 1
#endif
template <int W, int KVF, int SWF, bool FINAL>
__global__ __launch_bounds__(64 * W, W == 1 ? 1 : CSA2_ATTN_WAVES_PER_SIMD) void attend_kernel(AttnArgs a) {
  __shared__ AttnShared sh;
  const int item = blockIdx.x, t = blockIdx.y;
  const int layer = block_layer<W>(), hg = head_group<W>();
  const int b = t / a.q_per_seq;
  const int n_chunks = a.n_main + a.n_swa;
  const int c0 = item * a.cpw;
  const int c1 = c0 + a.cpw < n_chunks ? c0 + a.cpw : n_chunks;
  if (FINAL && a.rope_pos && threadIdx.x < 32) {
    float c, sn;
    rope_cs(a, t, threadIdx.x, &c, &sn);
    sh.rope[threadIdx.x][0] = c;
    sh.rope[threadIdx.x][1] = sn;
  }
  bf16x8 qb[16];
  HeadState st;
  if (W == 1) {
    stage_chunk<KVF, SWF>(a, sh, t, b, c0, layer);
    load_q(a, layer, t, hg, qb);
    state_init(st);
    __syncthreads();
    attend_chunk(a, sh, qb, st);
  } else {
    // wave hg stages row group hg; the next chunk's bytes are in flight
    // during this chunk's products
    int32_t idx[8];
    RawGroup rg;
    load_indices(a, t, c0, hg, idx);
    load_group_raw<KVF, SWF>(a, t, b, c0, layer, hg, idx, rg);
    if (c0 + 1 < c1) load_indices(a, t, c0 + 1, hg, idx);
    load_q(a, layer, t, hg, qb);
    state_init(st);
    for (int c = c0; c < c1; ++c) {
      store_group_raw<KVF, SWF>(a, sh, c, hg, rg);
      __syncthreads();
      if (c + 1 < c1) {
        load_group_raw<KVF, SWF>(a, t, b, c + 1, layer, hg, idx, rg);
        if (c + 2 < c1) load_indices(a, t, c + 2, hg, idx);
      }
      attend_chunk(a, sh, qb, st);
      __syncthreads();
    }
  }
  if (FINAL) write_final(a, sh, st, layer, t, hg);
  else write_partial(a, st, layer, t, item, hg);
}

// ---------------------------------------------------------------------------
// Eight-wave blocks: one query-layer per block, the work of a chunk split so
// that every wave touches only a slice of it and holds half a wave's worth of
// state (two waves per SIMD):
//   S^T = X Q^T: wave w takes heads 16 (w & 3) .. +15 over channels
//     256 (w >> 2) .. +255.  For selected rows the A operands are dequantised
//     from the chunk's raw bytes, which arrive in LDS by direct-to-LDS
//     requests (cs_issue_rows): lane (r, g) holds rows r and 16 + r, channels
//     256 (w >> 2) + 64 g .. +63, k-step j taking channels + 8 j .. + 8 (the
//     order of the channels along k does not change the products; the query
//     operand uses the same order).  Window chunks (bf16 or FP8 rows, four
//     times the bytes of FP4 ones) take them from a row-major copy in LDS.
//     The two channel halves of a head group exchange their partial S^T
//     through LDS (2 KB per wave); both form the head group's maximum and
//     rescale state, each the probabilities of its own 16 rows.
//   O^T += X^T P^T: wave w takes channels 64 w .. +63 of all 64 heads; its A
//     operand is its own transposed slice of the chunk in LDS (staged by the
//     wave itself), the B operand P^T of head group G comes from LDS, written
//     by the two waves of group G.  These products of a chunk run at the start
//     of the next chunk, ahead of its staging.

constexpr int kCsThreads = 512;
constexpr int kCsSlice = kDim / 8;  // output channels per wave

// The bytes of one selected-row chunk (the kernel keeps two, each an LDS
// object of its own, so that the compiler can tell the direct-to-LDS requests
// into one from every other LDS access).
struct CsRows {
  alignas(16) uint8_t rawc[kChunk * 256];  // E2M1 codes, 16-byte pieces swizzled (cs_piece)
  alignas(16) uint8_t raws[kChunk * 32];   // scales: 16 (MXFP4) or 32 (E4M3) bytes per row
};

struct CsShared {
  alignas(16) uint16_t xt[8][kCsSlice * kXTStride];  // per wave: channel c of its slice, 32 rows (k order)
  alignas(16) uint16_t x[kChunk * kXStride];          // window chunks: row-major rows (S operand)
  alignas(16) floatx4 sx[8][2][64];                   // partial S^T [wave][m-tile][lane]
  alignas(16) bf16x8 p[4][64];                        // P^T of head group G, B-operand layout
  float alpha[kHeads];                                // this chunk's rescale factor per head
  alignas(16) int grow[4];                            // head group G rescales this chunk
  float fin_m[kHeads], fin_l[kHeads][2];              // final max, and sum of each half's rows, per head
  float rope[32][2];
  int32_t idx[CSA2_TOPK];                             // the query's selected rows
};

// XT slice layout: row c (channel), four 16-byte blocks of 8 rows (k order),
// block b stored at position (b + c / 16) % 4: the O loop's reads (16
// consecutive channels, one block) hit 16 distinct bank groups.
__device__ __forceinline__ int cs_xt_off(int c, int blk) { return c * kXTStride + 8 * ((blk + (c >> 4)) & 3); }

// Maximum with the lane l ^ 16 / l ^ 32 (gfx950 lane swaps).
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Slice-layout rows of lane l: k-block l / 16 holds rows group_row(b, 0..7);
// lane l takes k positions 4 (l >> 3) .. +3, i.e. rows group_row(l >> 4,
// 4 ((l >> 3) & 1) + i), channels 64 w + 8 (l & 7) .. +7.
__device__ __forceinline__ int cs_slice_row(int lane, int i) { return group_row(lane >> 4, 4 * ((lane >> 3) & 1) + i); }

// Raw bytes of a window chunk for one wave, slice layout: x[i] for row
// cs_slice_row(lane, i) (the 16-byte piece, or FP8 code bytes and scale).
struct CsRaw {
  uint4 x[4];
  uint32_t ok;  // bit r: row r of the chunk valid (the same in every lane)
};

// Selected-row chunks go through LDS: a chunk's 32 rows are requested with
// one 16-byte piece per lane, each wave four whole rows of codes (whole cache
// lines per request, every byte requested once), wave 0 also the rows'
// scales, straight into LDS (global_load_lds_dwordx4: lane l's piece lands at
// the wave's base + 16 l); every wave then reads its operands from there.
// Piece p of row r sits in slot p ^ (r % 16), so that the sixteen rows an
// operand read spans fall in distinct bank groups.
__device__ __forceinline__ int cs_piece(int r, int p) { return r * 256 + 16 * (p ^ (r & 15)); }

template <int KVF>
__device__ __forceinline__ void cs_issue_rows(const AttnArgs& a, const CsShared& sh, CsRows& rw, int b, int c) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r = 4 * w + (lane >> 4);
  const int32_t e = sh.idx[c * kChunk + r];
  const size_t rowid = (size_t)b * a.N + (e >= 0 ? e : 0);  // invalid rows read row 0, masked later
  __builtin_amdgcn_global_load_lds(a.kv_fp4 + rowid * 256 + 16 * ((lane & 15) ^ (r & 15)), &rw.rawc[w * 1024],
                                   16, 0, 0);
  if (w == 0) {
    if (KVF == CSA2_KV_MXFP4) {
      if (lane < kChunk) {
        const int32_t es = sh.idx[c * kChunk + lane];
        __builtin_amdgcn_global_load_lds(a.kv_scale + ((size_t)b * a.N + (es >= 0 ? es : 0)) * 16, &rw.raws[0],
                                         16, 0, 0);
      }
    } else {
      const int32_t es = sh.idx[c * kChunk + (lane >> 1)];
      __builtin_amdgcn_global_load_lds(a.kv_scale + ((size_t)b * a.N + (es >= 0 ? es : 0)) * 32 + 16 * (lane & 1),
                                       &rw.raws[0], 16, 0, 0);
    }
  }
}

// Every vector-memory request of this wave done (the row staging included).
__device__ __forceinline__ void cs_wait_rows() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <int KVF, int SWF>
__device__ __forceinline__ void cs_load_raw(const AttnArgs& a, int t, int b, int c, int layer, CsRaw& raw) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int xc0 = kCsSlice * w + 8 * (lane & 7);  // slice-layout channels xc0 .. xc0 + 7
  const int we = a.swa_end[t];
  const int ws = we - a.window > 0 ? we - a.window : 0;
  const int row0 = ws + (c - a.n_main) * kChunk;
  const size_t base = ((size_t)layer * a.B + b) * a.S;
  const int last = we > 0 ? we - 1 : 0;
  const int nvalid = we - row0 < 0 ? 0 : (we - row0 > kChunk ? kChunk : we - row0);  // rows row0 .. we-1
  raw.ok = nvalid >= kChunk ? 0xFFFFFFFFu : (1u << nvalid) - 1u;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = row0 + cs_slice_row(lane, i);
    const size_t rr = base + (row < we ? row : last);
    if (SWF == CSA2_SWA_BF16) {
      raw.x[i] = *reinterpret_cast<const uint4*>(a.swa + rr * kDim + xc0);
    } else if (xc0 >= 448) {
      raw.x[i] = *reinterpret_cast<const uint4*>(a.swa_rope + rr * 64 + (xc0 - 448));
    } else {
      const uint2 cw = *reinterpret_cast<const uint2*>(a.swa_fp8 + rr * 448 + xc0);
      raw.x[i] = make_uint4(cw.x, cw.y, a.swa_sc[rr * 8 + xc0 / 64], 0u);
    }
  }
}

// The wave's transposed slice of a chunk into LDS (selected rows from `rw`,
// window rows from `raw`); for window chunks (WIN) also its part of the
// row-major copy.
template <int KVF, int SWF, bool WIN>
__device__ __forceinline__ void cs_store_slice(const AttnArgs& a, CsShared& sh, const CsRows& rw, const CsRaw& raw) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int cg = lane & 7, kb = lane >> 3;
  const int xc0 = kCsSlice * w + 8 * cg;
  const int q = 2 * w + (cg >> 2);  // code piece of channels xc0 .. xc0 + 7 (and their MXFP4 scale block)
  uint32_t v[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint4 o;
    if (!WIN) {
      const int r = cs_slice_row(lane, i);
      const uint32_t cw = *reinterpret_cast<const uint32_t*>(&rw.rawc[cs_piece(r, q) + 4 * (cg & 3)]);
      o = KVF == CSA2_KV_MXFP4 ? dequant8(cw, rw.raws[r * 16 + q]) : dequant8_e4m3(cw, rw.raws[r * 32 + 4 * w + (cg >> 1)]);
    } else if (SWF == CSA2_SWA_BF16 || xc0 >= 448) {
      o = raw.x[i];
    } else {
      const float sc = e8m0_f32(raw.x[i].z);
      o.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.x[i].x, sc, false));
      o.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.x[i].x, sc, true));
      o.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.x[i].y, sc, false));
      o.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.x[i].y, sc, true));
    }
    v[i][0] = o.x; v[i][1] = o.y; v[i][2] = o.z; v[i][3] = o.w;
  }
  if (WIN) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<uint4*>(&sh.x[cs_slice_row(lane, i) * kXStride + xc0]) =
          make_uint4(v[i][0], v[i][1], v[i][2], v[i][3]);
  }
  // channel 8 cg + e of the slice, k positions 4 kb .. 4 kb + 3
  uint16_t* xt = sh.xt[w];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    uint32_t wd[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const uint32_t lo = (v[2 * p][e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
      const uint32_t hi = (v[2 * p + 1][e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
      wd[p] = lo | (hi << 16);
    }
    *reinterpret_cast<uint2*>(&xt[cs_xt_off(8 * cg + e, kb >> 1) + 4 * (kb & 1)]) = make_uint2(wd[0], wd[1]);
  }
}

// S^T partial product of the wave's 16 heads over its 256 channels: A
// operands of selected-row chunks from the raw S-layout bytes, of window
// chunks from the row-major LDS copy (rows r and 16 + r, channels sc0 + 8 j).
template <int KVF, bool WIN>
__device__ __forceinline__ void cs_s_product(const CsShared& sh, const CsRows& rw, const bf16x8 (&qb)[8],
                                             floatx4 (&acc)[2], int sc0) {
  const int r16 = threadIdx.x & 15;
  acc[0] = floatx4{0.f, 0.f, 0.f, 0.f};
  acc[1] = floatx4{0.f, 0.f, 0.f, 0.f};
  // selected rows: lane (r, g) reads rows r and 16 + r, code pieces sc0 / 32 and + 1 (channels sc0 .. + 63)
  // and their scale bytes (two E8M0 or four E4M3)
  uint32_t cw[2][8], ss[2];
  if (!WIN) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int r = 16 * m + r16;
      const uint4 c0 = *reinterpret_cast<const uint4*>(&rw.rawc[cs_piece(r, sc0 / 32)]);
      const uint4 c1 = *reinterpret_cast<const uint4*>(&rw.rawc[cs_piece(r, sc0 / 32 + 1)]);
      cw[m][0] = c0.x; cw[m][1] = c0.y; cw[m][2] = c0.z; cw[m][3] = c0.w;
      cw[m][4] = c1.x; cw[m][5] = c1.y; cw[m][6] = c1.z; cw[m][7] = c1.w;
      ss[m] = KVF == CSA2_KV_MXFP4 ? (uint32_t)*reinterpret_cast<const uint16_t*>(&rw.raws[r * 16 + sc0 / 32])
                                   : *reinterpret_cast<const uint32_t*>(&rw.raws[r * 32 + sc0 / 16]);
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      bf16x8 av;
      if (WIN) {
        av = lds_read16(&sh.x[(16 * m + r16) * kXStride + sc0 + 8 * j]);
      } else {
        const uint32_t sb = KVF == CSA2_KV_MXFP4 ? (ss[m] >> (8 * (j >> 2))) & 255u : (ss[m] >> (8 * (j >> 1))) & 255u;
        av = as_bf16x8(KVF == CSA2_KV_MXFP4 ? dequant8(cw[m][j], sb) : dequant8_e4m3(cw[m][j], sb));
      }
      acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, qb[j], acc[m], 0, 0, 0);
    }
  }
}

struct CsState {
  floatx4 o[4][4];  // O^T: o[mb][G][i] = O[16 G + lane % 16][64 w + 16 mb + 4 (lane / 16) + i]
  float m;          // running max (log2 units) of head 16 (w & 3) + lane % 16
  float l;          // running sum over this lane's rows
};

template <bool B>
struct CsFlag {
  static constexpr bool value = B;
};

// grid (n_items, T, L), 512 threads; chunks and outputs as attend_kernel.
template <int KVF, int SWF, bool FINAL>
__global__ __launch_bounds__(kCsThreads) void attend_cs_kernel(AttnArgs a) {
  __shared__ CsShared sh;
  __shared__ CsRows rows0, rows1;
  const int item = blockIdx.x, t = blockIdx.y, layer = blockIdx.z;
  const int b = t / a.q_per_seq;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4, hg = w & 3, h = w >> 2;
  const int sc0 = 256 * h + 64 * g;
  const int n_chunks = a.n_main + a.n_swa;
  const int c0 = item * a.cpw;
  const int c1 = c0 + a.cpw < n_chunks ? c0 + a.cpw : n_chunks;
  if (FINAL && a.rope_pos && threadIdx.x < 32) {
    float cv, sv;
    rope_cs(a, t, threadIdx.x, &cv, &sv);
    sh.rope[threadIdx.x][0] = cv;
    sh.rope[threadIdx.x][1] = sv;
  }
  // the query's selected rows (one coalesced load), then the first chunk's bytes
  for (int i = threadIdx.x; i < a.n_main * kChunk; i += kCsThreads) sh.idx[i] = a.indices[(size_t)t * a.k + i];
  __syncthreads();
  CsRaw raw;
  if (c0 < a.n_main) cs_issue_rows<KVF>(a, sh, rows0, b, c0);
  else cs_load_raw<KVF, SWF>(a, t, b, c0, layer, raw);
  // the query operand: head 16 hg + r16, channels sc0 + 8 j .. + 8
  bf16x8 qb[8];
  {
    const uint4* qp = reinterpret_cast<const uint4*>(
        a.q + (((size_t)layer * a.T + t) * kHeads + 16 * hg + r16) * kDim + sc0);
#pragma unroll
    for (int j = 0; j < 8; ++j) qb[j] = as_bf16x8(qp[j]);
  }
  CsState st;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int G = 0; G < 4; ++G) st.o[mb][G] = floatx4{0.f, 0.f, 0.f, 0.f};
  st.m = -INFINITY;
  st.l = 0.f;
  // The rows of selected-row chunk c are requested two chunks ahead, into the
  // buffer chunk c - 2 used (consumed before the barrier that precedes the
  // request), and every wave waits for its own requests before the barrier
  // ahead of the chunk; window chunks are loaded into registers one chunk ahead.
  cs_wait_rows();
  __syncthreads();
  if (c0 + 1 < c1 && c0 + 1 < a.n_main) cs_issue_rows<KVF>(a, sh, rows1, b, c0 + 1);

  // O^T of the previous chunk, all four head groups of this wave's channels:
  // its slice in sh.xt (this wave's own), its P^T, rescale factors and flags
  // from that chunk's softmax (the first chunk's rescale multiplies zeros).
  const auto o_phase = [&]() {
    const int4 grows = *reinterpret_cast<const int4*>(sh.grow);
    const int grw[4] = {grows.x, grows.y, grows.z, grows.w};
#pragma unroll
    for (int G = 0; G < 4; ++G) {
      if (grw[G]) {
        const float al = sh.alpha[16 * G + r16];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) st.o[mb][G] *= al;
      }
    }
    bf16x8 xa[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) xa[mb] = lds_read16(&sh.xt[w][cs_xt_off(16 * mb + r16, g)]);
#pragma unroll
    for (int G = 0; G < 4; ++G) {
      const bf16x8 pv = sh.p[G][lane];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) st.o[mb][G] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[mb], pv, st.o[mb][G], 0, 0, 0);
    }
  };

  // One chunk c: the previous chunk's O^T (none before the item's first
  // chunk), this chunk's slice and S^T, its softmax.  Selected rows (WIN
  // false) come from `cur`, which then receives chunk c + 2; window rows from
  // `raw`, loaded one chunk ahead.  The O^T products overlap this chunk's
  // staging: the two need different units.
  const auto chunk = [&](auto win, auto first, int c, CsRows& cur) {
      constexpr bool WIN = decltype(win)::value;
      if (!decltype(first)::value) o_phase();
      cs_store_slice<KVF, SWF, WIN>(a, sh, cur, raw);
      uint32_t ok;  // this chunk's valid rows
      floatx4 acc[2];
      if (!WIN) {
        ok = (uint32_t)__ballot(lane < kChunk && sh.idx[c * kChunk + (lane & (kChunk - 1))] >= 0);
        cs_s_product<KVF, false>(sh, cur, qb, acc, sc0);
      } else {
        ok = __builtin_amdgcn_readfirstlane(raw.ok);
        __syncthreads();  // the window rows of every wave in sh.x
        cs_s_product<KVF, true>(sh, cur, qb, acc, sc0);
      }
      // each half's partial S, for both halves' softmax
      sh.sx[w][0][lane] = acc[0];
      sh.sx[w][1][lane] = acc[1];
      if (c + 1 < c1 && c + 1 >= a.n_main) cs_load_raw<KVF, SWF>(a, t, b, c + 1, layer, raw);
      __syncthreads();
      // Softmax of head group hg: both halves form the full S^T (own + partner
      // partial, the same sums in either order) and the same maximum and
      // rescale state; half h forms the probabilities of rows 16 h + 4 g + i
      // and keeps the sum of its own rows.
      {
        acc[0] += sh.sx[w ^ 4][0][lane];
        acc[1] += sh.sx[w ^ 4][1][lane];
        // acc[m][i]: row 16 m + 4 g + i, head 16 hg + r16
        float z[8];
        if (ok == 0xFFFFFFFFu) {
  #pragma unroll
          for (int i = 0; i < 4; ++i) {
            z[i] = acc[0][i] * a.scale_log2;
            z[4 + i] = acc[1][i] * a.scale_log2;
          }
        } else {
          const uint32_t okg = ok >> (4 * g);
  #pragma unroll
          for (int i = 0; i < 4; ++i) {
            z[i] = ((okg >> i) & 1u) ? acc[0][i] * a.scale_log2 : -INFINITY;
            z[4 + i] = ((okg >> (16 + i)) & 1u) ? acc[1][i] * a.scale_log2 : -INFINITY;
          }
        }
        float cm = fmaxf(fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3])), fmaxf(fmaxf(z[4], z[5]), fmaxf(z[6], z[7])));
        cm = max_xor16(cm);
        cm = max_xor32(cm);
        // lazy rescaling: the reference maximum stays while the chunk's scores
        // exceed it by at most kRescaleSlack (log2 units)
        const float mtrue = fmaxf(st.m, cm);
        const bool grow = mtrue > st.m + kRescaleSlack;
        const float mn = grow ? mtrue : st.m;
        const float alpha = grow ? exp2f(st.m - mn) : 1.f;
        // 2^(z - mn) by v_exp_f32 (masked scores -inf give 0; mn is -inf only
        // while every score so far is masked)
        const float mref = mn == -INFINITY ? 0.f : mn;
        float p[4];
  #pragma unroll
        for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f((h == 0 ? z[i] : z[4 + i]) - mref);
        st.l = st.l * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
        st.m = mn;
        reinterpret_cast<u32x2*>(&sh.p[hg][lane])[h] = u32x2{pack_bf16x2_rne(p[0], p[1]), pack_bf16x2_rne(p[2], p[3])};
        const bool any = __ballot(grow) != 0ull;
        if (h == 0) {
          if (g == 0) sh.alpha[16 * hg + r16] = alpha;
          if (lane == 0) sh.grow[hg] = any ? 1 : 0;
        }
      }
      if (!WIN) cs_wait_rows();  // the next chunk's rows (requested a chunk ago) are in LDS
      __syncthreads();
      if (!WIN && c + 2 < c1 && c + 2 < a.n_main) cs_issue_rows<KVF>(a, sh, cur, b, c + 2);
  };
  // selected-row chunks alternate between rows0 and rows1 (chunk c0 + i in
  // rows0 for even i; two LDS objects: the requests into one never make the
  // compiler wait before reads of the other), then the window chunks
  const int cs_end = c1 < a.n_main ? c1 : a.n_main;
  int c = c0;
  if (c < cs_end) chunk(CsFlag<false>(), CsFlag<true>(), c++, rows0);
  else chunk(CsFlag<true>(), CsFlag<true>(), c++, rows0);
  for (; c + 1 < cs_end; c += 2) {
    chunk(CsFlag<false>(), CsFlag<false>(), c, rows1);
    chunk(CsFlag<false>(), CsFlag<false>(), c + 1, rows0);
  }
  if (c < cs_end) chunk(CsFlag<false>(), CsFlag<false>(), c++, rows1);
  for (; c < c1; ++c) chunk(CsFlag<true>(), CsFlag<false>(), c, rows0);
  o_phase();
  // max of each head (the same in both halves), sum of each half's rows
  {
    float l = st.l;
    l = sum_xor16(l);
    l = sum_xor32(l);
    if (g == 0) {
      if (h == 0) sh.fin_m[16 * hg + r16] = st.m;
      sh.fin_l[16 * hg + r16][h] = l;
    }
  }
  __syncthreads();
  const size_t qrow = ((size_t)layer * a.T + t) * kHeads;
#pragma unroll
  for (int G = 0; G < 4; ++G) {
    const int head = 16 * G + r16;
    float m = sh.fin_m[head];
    const float l = sh.fin_l[head][0] + sh.fin_l[head][1];
    if (FINAL) {
      float den = l, f = 1.f;
      if (a.sink) {
        const float sk = a.sink[(size_t)layer * kHeads + head] * kLog2e;
        const float M = fmaxf(m, sk);
        if (M != -INFINITY) {
          f = (m == -INFINITY) ? 0.f : exp2f(m - M);
          den = l * f + exp2f(sk - M);
          m = M;
        }
      }
      const float inv = (m == -INFINITY || den == 0.f) ? 0.f : f / den;
      uint16_t* op = a.out + (qrow + head) * kDim + kCsSlice * w + 4 * g;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        float v[4] = {st.o[mb][G][0] * inv, st.o[mb][G][1] * inv, st.o[mb][G][2] * inv, st.o[mb][G][3] * inv};
        if (w == 7 && a.rope_pos) {  // channels 448..511: pairs (v0, v1), (v2, v3)
          const int j0 = 8 * mb + 2 * g;
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            const float cv = sh.rope[j0 + p][0], sv = sh.rope[j0 + p][1];
            const float x = v[2 * p], y = v[2 * p + 1];
            v[2 * p] = x * cv - y * sv;
            v[2 * p + 1] = x * sv + y * cv;
          }
        }
        *reinterpret_cast<uint2*>(op + 16 * mb) = make_uint2(pack_bf16x2_rne(v[0], v[1]), pack_bf16x2_rne(v[2], v[3]));
      }
      if (a.lse && w == 0 && g == 0)
        a.lse[qrow + head] = (m == -INFINITY) ? -INFINITY : (m + log2f(den)) * kLn2;
    } else {
      const size_t slot_id = ((size_t)layer * a.T + t) * a.n_items + item;
      const size_t base = slot_id * kHeads + head;
      uint16_t* op = a.part_o + slot_id * kHeads * kDim + part_tile_off(G, 4 * w, r16, 4 * g);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const u32x2 wv = {pack_bf16x2_rne(st.o[mb][G][0], st.o[mb][G][1]),
                          pack_bf16x2_rne(st.o[mb][G][2], st.o[mb][G][3])};
        __builtin_nontemporal_store(wv, reinterpret_cast<u32x2*>(op + 256 * mb));
      }
      if (w == 0 && g == 0) {
        a.part_ml[base * 2 + 0] = m;
        a.part_ml[base * 2 + 1] = l;
      }
    }
  }
}

// Merge the partial slots of each (layer, query): block (32 G + ct, t, layer),
// one wave, takes partial tile ct of head group G (heads 16G .. 16G+15,
// channels 16ct .. 16ct+15).  out = sum_s O_s 2^(m_s - M) / den,
// den = sum_s l_s 2^(m_s - M) (+ 2^(sink - M)), M = max_s m_s (and the sink).
// Lane (r, g) takes head 16G + r, channels 16ct + 4g .. +3: each slot's tile
// read is 512 contiguous bytes, and all slots' loads are issued before any is
// used.  Small blocks spread the reads over every CU: the kernel is bound by
// how many cache lines each CU can have in flight at small T.
__global__ __launch_bounds__(64) void attend_combine_kernel(AttnArgs a) {
  const int G = blockIdx.x >> 5, ct = blockIdx.x & 31, t = blockIdx.y, layer = blockIdx.z;
  const int lane = threadIdx.x, r = lane >> 2, g = lane & 3;
  const int head = 16 * G + r;
  const int n = a.n_items;
  const size_t slot0 = ((size_t)layer * a.T + t) * n;
  const size_t toff = part_tile_off(G, ct, r, 4 * g);
  float2 ml[kMaxSlots];
  uint2 v[kMaxSlots];
#pragma unroll
  for (int s = 0; s < kMaxSlots; ++s)
    if (s < n) {
      ml[s] = *reinterpret_cast<const float2*>(a.part_ml + ((slot0 + s) * kHeads + head) * 2);
      v[s] = *reinterpret_cast<const uint2*>(a.part_o + (slot0 + s) * kHeads * kDim + toff);
    }
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < kMaxSlots; ++s)
    if (s < n) M = fmaxf(M, ml[s].x);
  float sk = -INFINITY;
  if (a.sink) {
    sk = a.sink[(size_t)layer * kHeads + head] * kLog2e;
    M = fmaxf(M, sk);
  }
  float den = 0.f;
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < kMaxSlots; ++s)
    if (s < n) {
      const float f = (M == -INFINITY || ml[s].x == -INFINITY) ? 0.f : exp2f(ml[s].x - M);
      if (f != 0.f) {
        den += ml[s].y * f;
        const floatx4 x = {bf16lo(v[s].x), bf16hi(v[s].x), bf16lo(v[s].y), bf16hi(v[s].y)};
        acc += x * f;
      }
    }
  if (a.sink && M != -INFINITY) den += exp2f(sk - M);
  const float inv = (M == -INFINITY || den == 0.f) ? 0.f : 1.f / den;
  if (a.lse && ct == 0 && g == 0)
    a.lse[((size_t)layer * a.T + t) * kHeads + head] = (M == -INFINITY) ? -INFINITY : (M + log2f(den)) * kLn2;
  float x[4] = {acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
  if (ct >= 28 && a.rope_pos) {  // channels 448..511: pairs (x0, x1), (x2, x3)
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      float cv, sv;
      rope_cs(a, t, 8 * (ct - 28) + 2 * g + p, &cv, &sv);
      const float x0 = x[2 * p], x1 = x[2 * p + 1];
      x[2 * p] = x0 * cv - x1 * sv;
      x[2 * p + 1] = x0 * sv + x1 * cv;
    }
  }
  uint16_t* op = a.out + (((size_t)layer * a.T + t) * kHeads + head) * kDim + 16 * ct + 4 * g;
  *reinterpret_cast<uint2*>(op) = make_uint2(pack_bf16x2_rne(x[0], x[1]), pack_bf16x2_rne(x[2], x[3]));
}

struct AttendPlan {
  int n_main, n_swa, cpw, n_items;
};

// One-wave blocks (a work item's four head groups on four CUs) while the
// whole launch fits in one round of them (two per CU, by their LDS).
constexpr int kOneWaveBlocks = 512;

// Cost model of a split, fitted to timings of these kernels on MI355X
// (256 CUs).  The eight-wave blocks run one per CU (their LDS), so Q
// query-layers split into n work items of cpw chunks take ceil(Q n / 256)
// rounds of cpw chunks, about 3.3 us per chunk; a split (n > 1) adds the
// combine launch, about 4 us, and a 64 KiB partial per work item, written
// and read back at about 4 TB/s.
constexpr int kPlanCUs = 256;
constexpr double kPlanChunkUs = 3.3;
constexpr double kPlanCombineUs = 4.0;
constexpr double kPlanSlotUs = (kHeads * kDim * 2.0) * 2.0 / 4.0e6;  // 64 KiB out and back at 4 TB/s

// The split of each query-layer's chunks over work items for a launch of T
// query rows x L layers: the item count of least modelled time (ties to
// fewer items, i.e. less partial traffic).  Launches with at least one
// query-layer per CU are not split: every CU already has a block.  A
// query-layer's result depends on the split only through the rounding of the
// merge, so the same rows can round differently in launches of other shapes.
static AttendPlan attend_plan(int32_t T, int32_t L, int32_t k, int32_t window) {
  AttendPlan p;
  p.n_main = (k + kChunk - 1) / kChunk;
  p.n_swa = (window + kChunk - 1) / kChunk;
  const int n_chunks = p.n_main + p.n_swa;
  const int64_t Q = (int64_t)T * L;
  p.cpw = n_chunks;
  p.n_items = 1;
  if (Q >= kPlanCUs) return p;
  double best = 0.0;
  // cpw downwards: n grows, and of the cpw giving the same n the last (least) costs least
  for (int cpw = n_chunks; cpw >= 1; --cpw) {
    const int n = (n_chunks + cpw - 1) / cpw;
    const double rounds = (double)((Q * n + kPlanCUs - 1) / kPlanCUs);
    const double cost = rounds * cpw * kPlanChunkUs + (n == 1 ? 0.0 : kPlanCombineUs + (double)Q * n * kPlanSlotUs);
    if (cpw == n_chunks || cost < best - 1e-9) {
      best = cost;
      p.cpw = cpw;
      p.n_items = n;
    }
  }
  return p;
}

static size_t attend_ws_bytes(int32_t T, const AttendPlan& p, int32_t L) {
  if (p.n_items == 1) return 0;
  const size_t slots = (size_t)L * T * p.n_items;
  return align_up(slots * kHeads * kDim * sizeof(uint16_t), 256) + align_up(slots * kHeads * 2 * sizeof(float), 256);
}

static csa2_status attend_launch(int32_t L, const void* q, const uint8_t* kv_fp4, const uint8_t* kv_scale,
                                 const int32_t* indices, const void* swa, const int32_t* swa_end,
                                 const float* sink, float softmax_scale, int32_t T, int32_t q_per_seq,
                                 int64_t N, int32_t S, int32_t window, int32_t k, const csa2_attend_opts* opts,
                                 void* out, float* lse, void* workspace, size_t workspace_bytes, void* hip_stream) {
  const csa2_attend_opts o = opts ? *opts : csa2_attend_opts{};
  if (o.kv_format != CSA2_KV_MXFP4 && o.kv_format != CSA2_KV_E4M3_16) return CSA2_ERR_UNSUPPORTED;
  if (o.swa_format != CSA2_SWA_BF16 && o.swa_format != CSA2_SWA_FP8) return CSA2_ERR_UNSUPPORTED;
  const bool fp8w = o.swa_format == CSA2_SWA_FP8;
  if (!q || !kv_fp4 || !kv_scale || !indices || !swa_end || !out) return CSA2_ERR_INVALID_ARG;
  if (fp8w ? (!o.swa_fp8 || !o.swa_rope || !o.swa_scales) : !swa) return CSA2_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(kv_fp4) || !aligned16(kv_scale) || !aligned16(indices) ||
      (!fp8w && !aligned16(swa)) ||
      (fp8w && (!aligned16(o.swa_fp8) || !aligned16(o.swa_rope) || !aligned16(o.swa_scales))) ||
      !aligned16(swa_end) || !aligned16(out) || (sink && !aligned16(sink)) || (lse && !aligned16(lse)) ||
      (o.rope_pos && !aligned16(o.rope_pos)))
    return CSA2_ERR_INVALID_ARG;
  if (o.rope_pos && !(o.rope_base > 1.f && o.rope_base < INFINITY)) return CSA2_ERR_INVALID_ARG;
  if (T < 1 || q_per_seq < 1 || T % q_per_seq != 0 || N < 1 || S < 1) return CSA2_ERR_INVALID_ARG;
  if (!(softmax_scale > 0.f) || !(softmax_scale < INFINITY)) return CSA2_ERR_INVALID_ARG;
  if (k != kTopK || window < 1 || window > CSA2_MAX_WINDOW || L < 1 || L > CSA2_MAX_LAYERS || T > 65535 ||
      N >= ((int64_t)1 << 31))
    return CSA2_ERR_UNSUPPORTED;
  const AttendPlan p = attend_plan(T, L, k, window);
  const size_t need = attend_ws_bytes(T, p, L);
  if (need > 0 && (!workspace || !aligned16(workspace) || workspace_bytes < need)) return CSA2_ERR_WORKSPACE;
  AttnArgs a;
  a.q = (const uint16_t*)q;
  a.kv_fp4 = kv_fp4;
  a.kv_scale = kv_scale;
  a.indices = indices;
  a.swa = fp8w ? nullptr : (const uint16_t*)swa;
  a.swa_fp8 = fp8w ? o.swa_fp8 : nullptr;
  a.swa_rope = fp8w ? (const uint16_t*)o.swa_rope : nullptr;
  a.swa_sc = fp8w ? o.swa_scales : nullptr;
  a.rope_pos = o.rope_pos;
  a.rope_log2_base = o.rope_pos ? log2((double)o.rope_base) : 0.0;
  a.swa_end = swa_end;
  a.sink = sink;
  a.scale_log2 = softmax_scale * kLog2e;
  a.T = T;
  a.q_per_seq = q_per_seq;
  a.B = T / q_per_seq;
  a.S = S;
  a.window = window;
  a.k = k;
  a.L = L;
  a.N = N;
  a.n_main = p.n_main;
  a.n_swa = p.n_swa;
  a.cpw = p.cpw;
  a.n_items = p.n_items;
  a.out = (uint16_t*)out;
  a.lse = lse;
  const size_t slots = (size_t)L * T * p.n_items;
  a.part_o = need ? (uint16_t*)workspace : nullptr;
  a.part_ml = need ? (float*)((char*)workspace + align_up(slots * kHeads * kDim * sizeof(uint16_t), 256)) : nullptr;
  hipStream_t st = (hipStream_t)hip_stream;
  (void)hipGetLastError();
  // small launches: one wave per block and four blocks per work item (16
  // heads each), so that the work and the partial writes spread over four
  // times the CUs; otherwise four-wave blocks that stage each chunk once
  const bool one = p.cpw == 1 && (int64_t)L * T * p.n_items * 4 <= kOneWaveBlocks;
  const bool fin = p.n_items == 1;
  const dim3 grid(p.n_items, T, one ? 4 * L : L), block(one ? 64 : kCsThreads);
  const int fmt = 2 * o.kv_format + o.swa_format;
#define CSA2_ATTEND1(KVF, SWF) hipLaunchKernelGGL((attend_kernel<1, KVF, SWF, false>), grid, block, 0, st, a)
#define CSA2_ATTEND4(KVF, SWF, F) hipLaunchKernelGGL((attend_cs_kernel<KVF, SWF, F>), grid, block, 0, st, a)
#define CSA2_ATTEND_FMT(M, ...)                 \
  do {                                          \
    if (fmt == 0) M(0, 0 __VA_ARGS__);          \
    else if (fmt == 1) M(0, 1 __VA_ARGS__);     \
    else if (fmt == 2) M(1, 0 __VA_ARGS__);     \
    else M(1, 1 __VA_ARGS__);                   \
  } while (0)
  if (one) CSA2_ATTEND_FMT(CSA2_ATTEND1);
  else if (fin) CSA2_ATTEND_FMT(CSA2_ATTEND4, , true);
  else CSA2_ATTEND_FMT(CSA2_ATTEND4, , false);
#undef CSA2_ATTEND_FMT
#undef CSA2_ATTEND4
#undef CSA2_ATTEND1
  if (need) hipLaunchKernelGGL(attend_combine_kernel, dim3(4 * (kDim / 16), T, L), dim3(64), 0, st, a);
  if (hipGetLastError() != hipSuccess) return CSA2_ERR_LAUNCH;
  return CSA2_OK;
}

// ---- csa2_reuse_attend_static: the split-K partials in a file-scope device
// array instead of a caller's workspace.  Each GPU the library runs on holds
// its own copy until the process ends.  In host code the array's name is a
// host-side stand-in, never a device address: each device's address is looked
// up once (hipGetSymbolAddress, with that device current) and only that
// pointer reaches kernels.  Every slot a call reads was written by the same
// call, so nothing in the array needs clearing between calls; calls that
// overlap on one GPU race on it.
constexpr size_t kStaticScratchBytes = CSA2_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];
constexpr int kMaxStaticDevices = 64;
static void* g_scratch_ptr[kMaxStaticDevices];
static std::mutex g_scratch_mu;

// Device address of `scratch` on device dev (looked up on first use), or null.
static void* static_scratch(int dev) {
  if (dev < 0 || dev >= kMaxStaticDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return nullptr;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess || p == nullptr) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace csa2

using namespace csa2;

extern "C" size_t csa2_attend_workspace_bytes(int32_t T, int32_t k, int32_t window, int32_t n_layers) {
  if (T < 1 || k != kTopK || window < 1 || window > CSA2_MAX_WINDOW || n_layers < 1 || n_layers > CSA2_MAX_LAYERS)
    return 0;
  const AttendPlan p = attend_plan(T, n_layers, k, window);
  return attend_ws_bytes(T, p, n_layers);
}

extern "C" csa2_status csa2_attend_fp4(const void* q, const uint8_t* kv_fp4, const uint8_t* kv_scale,
                                       const int32_t* indices, const void* swa, const int32_t* swa_end,
                                       const float* sink, float softmax_scale, int32_t T, int32_t q_per_seq,
                                       int64_t N, int32_t S, int32_t window, int32_t k, void* out, float* lse,
                                       void* workspace, size_t workspace_bytes, void* hip_stream) {
  return attend_launch(1, q, kv_fp4, kv_scale, indices, swa, swa_end, sink, softmax_scale, T, q_per_seq, N, S,
                       window, k, nullptr, out, lse, workspace, workspace_bytes, hip_stream);
}

extern "C" csa2_status csa2_reuse_attend(int32_t n_layers, const void* q, const uint8_t* kv_fp4,
                                         const uint8_t* kv_scale, const int32_t* indices, const void* swa,
                                         const int32_t* swa_end, const float* sink, float softmax_scale,
                                         int32_t T, int32_t q_per_seq, int64_t N, int32_t S, int32_t window,
                                         int32_t k, void* out, float* lse, void* workspace, size_t workspace_bytes,
                                         void* hip_stream) {
  if (n_layers < 1 || n_layers > CSA2_MAX_LAYERS) return CSA2_ERR_UNSUPPORTED;
  return attend_launch(n_layers, q, kv_fp4, kv_scale, indices, swa, swa_end, sink, softmax_scale, T, q_per_seq, N,
                       S, window, k, nullptr, out, lse, workspace, workspace_bytes, hip_stream);
}

extern "C" csa2_status csa2_attend_ex(int32_t n_layers, const void* q, const uint8_t* kv_codes, const uint8_t* kv_scales,
                                      const int32_t* indices, const void* swa, const int32_t* swa_end,
                                      const float* sink, float softmax_scale, int32_t T, int32_t q_per_seq, int64_t N,
                                      int32_t S, int32_t window, int32_t k, const csa2_attend_opts* opts, void* out,
                                      float* lse, void* workspace, size_t workspace_bytes, void* hip_stream) {
  if (n_layers < 1 || n_layers > CSA2_MAX_LAYERS) return CSA2_ERR_UNSUPPORTED;
  return attend_launch(n_layers, q, kv_codes, kv_scales, indices, swa, swa_end, sink, softmax_scale, T, q_per_seq,
                       N, S, window, k, opts, out, lse, workspace, workspace_bytes, hip_stream);
}

extern "C" csa2_status csa2_reuse_attend_static(int32_t n_layers, const void* q, const uint8_t* kv_fp4,
                                                const uint8_t* kv_scale, const int32_t* indices, const void* swa,
                                                const int32_t* swa_end, const float* sink, float softmax_scale,
                                                int32_t T, int32_t q_per_seq, int64_t N, int32_t S, int32_t window,
                                                int32_t k, void* out, float* lse, void* hip_stream) {
  if (n_layers < 1 || n_layers > CSA2_MAX_LAYERS) return CSA2_ERR_UNSUPPORTED;
  // the size check comes first: nothing touches a device for a call that cannot fit
  if (T >= 1 && k == kTopK && window >= 1 && window <= CSA2_MAX_WINDOW &&
      csa2_attend_workspace_bytes(T, k, window, n_layers) > kStaticScratchBytes)
    return CSA2_ERR_WORKSPACE;
  if (!q || !kv_fp4 || !kv_scale || !indices || !swa || !swa_end || !out) return CSA2_ERR_INVALID_ARG;
  int dev = -1;
  const hipError_t e = hip_stream ? hipStreamGetDevice((hipStream_t)hip_stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return CSA2_ERR_LAUNCH;
  void* ws = static_scratch(dev);
  if (ws == nullptr) return CSA2_ERR_LAUNCH;
  return attend_launch(n_layers, q, kv_fp4, kv_scale, indices, swa, swa_end, sink, softmax_scale, T, q_per_seq, N,
                       S, window, k, nullptr, out, lse, ws, kStaticScratchBytes, hip_stream);
}
