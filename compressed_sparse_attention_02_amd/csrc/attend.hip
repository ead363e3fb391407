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
// sum, O) are merged by a combine kernel.  For Reuse with several layers,
// each selected-row chunk is staged once and used by every layer.
#include "mxfp4.h"

namespace csa2 {

constexpr int kAttnThreads = 256;
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
  int cpw;                  // chunks per work item (single layer)
  int n_items;              // work items per query
  int n_slots;              // partial slots per (layer, query)
  uint16_t* out;            // [L][T][64][512]
  float* lse;               // [L][T][64] or null
  uint16_t* part_o;         // [L][T][n_slots][64][512], bf16
  float* part_ml;           // [L][T][n_slots][64][2]  (max in log2 units, sum)
};

struct AttnShared {
  alignas(16) uint16_t X[kChunk * kXStride];
  alignas(16) uint16_t XT[kDim * kXTStride];
  int valid[kChunk];
  float rope[32][2];  // (cos, sin) of the output rotation of pair j (final outputs written here)
};

// Wave index over the 64 heads (16 heads per wave): a block of W waves takes
// head group blockIdx.z (grids with W = 1 split a work item's heads over four
// blocks).
__device__ __forceinline__ int head_wave() { return (int)(blockIdx.z * (blockDim.x >> 6) + (threadIdx.x >> 6)); }

// Two fp32 values rounded to nearest-even bf16 and packed, lo in the low half
// (one v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2_rne(float lo, float hi) {
  const __bf16 a = (__bf16)lo, b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
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

__device__ __forceinline__ void load_q(const AttnArgs& a, int layer, int t, bf16x8* qb) {
  const int lane = threadIdx.x & 63;
  const int head = 16 * head_wave() + (lane & 15), g = lane >> 4;
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
__device__ void write_final(const AttnArgs& a, const AttnShared& sh, const HeadState& st, int layer, int t) {
  const int lane = threadIdx.x & 63;
  const int head = 16 * head_wave() + (lane & 15), g = lane >> 4;
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

__device__ void write_partial(const AttnArgs& a, const HeadState& st, int layer, int t, int slot) {
  const int lane = threadIdx.x & 63;
  const int head = 16 * head_wave() + (lane & 15), g = lane >> 4;
  float l = st.l;
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  const size_t base = (((size_t)layer * a.T + t) * a.n_slots + slot) * kHeads + head;
  uint16_t* op = a.part_o + base * kDim + 4 * g;
  // bf16 partials (the combine accumulates in fp32); streaming stores: they
  // are read once, by the combine kernel
#pragma unroll
  for (int mb = 0; mb < 32; ++mb) {
    const uint32_t w0 = pack_bf16x2_rne(st.o[mb][0], st.o[mb][1]);
    const uint32_t w1 = pack_bf16x2_rne(st.o[mb][2], st.o[mb][3]);
    const u32x2 w = {w0, w1};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x2*>(op + 16 * mb));
  }
  if (g == 0) {
    a.part_ml[base * 2 + 0] = st.m;
    a.part_ml[base * 2 + 1] = l;
  }
}

// grid (n_items, T).  Work item i of query t:
//   L == 1: chunks [i*cpw, min((i+1)*cpw, n_main+n_swa)); if n_items == 1 the
//           result is final, otherwise it is partial slot i.
//   L  > 1: i < n_main: selected-row chunk i for every layer (slot i);
//           otherwise window chunk j of layer l, i = n_main + l*n_swa + j
//           (slot n_main + j of layer l).
template <int W, int KVF, int SWF>
__global__ __launch_bounds__(64 * W) void attend_kernel(AttnArgs a) {
  __shared__ AttnShared sh;
  const int item = blockIdx.x, t = blockIdx.y;
  const int b = t / a.q_per_seq;
  bf16x8 qb[16];
  HeadState st;
  if (a.L == 1) {
    const int n_chunks = a.n_main + a.n_swa;
    const int c0 = item * a.cpw;
    const int c1 = c0 + a.cpw < n_chunks ? c0 + a.cpw : n_chunks;
    if (a.n_items == 1 && a.rope_pos && threadIdx.x < 32) {
      float c, sn;
      rope_cs(a, t, threadIdx.x, &c, &sn);
      sh.rope[threadIdx.x][0] = c;
      sh.rope[threadIdx.x][1] = sn;
    }
    load_q(a, 0, t, qb);
    state_init(st);
    for (int c = c0; c < c1; ++c) {
      stage_chunk<KVF, SWF>(a, sh, t, b, c, 0);
      __syncthreads();
      attend_chunk(a, sh, qb, st);
      __syncthreads();
    }
    if (a.n_items == 1) write_final(a, sh, st, 0, t);
    else write_partial(a, st, 0, t, item);
  } else if (item < a.n_main) {
    stage_chunk<KVF, SWF>(a, sh, t, b, item, 0);
    __syncthreads();
    for (int l = 0; l < a.L; ++l) {
      load_q(a, l, t, qb);
      state_init(st);
      attend_chunk(a, sh, qb, st);
      write_partial(a, st, l, t, item);
    }
  } else {
    const int rest = item - a.n_main;
    const int l = rest / a.n_swa, j = rest % a.n_swa;
    load_q(a, l, t, qb);
    state_init(st);
    stage_chunk<KVF, SWF>(a, sh, t, b, a.n_main + j, l);
    __syncthreads();
    attend_chunk(a, sh, qb, st);
    write_partial(a, st, l, t, a.n_main + j);
  }
}

// Merge the partial slots of each (layer, query, head): grid (64, T, L),
// 128 threads x 4 channels.  out = sum_s O_s 2^(m_s - M) / den,
// den = sum_s l_s 2^(m_s - M) (+ 2^(sink - M)), M = max_s m_s (and the sink).
__global__ __launch_bounds__(128) void attend_combine_kernel(AttnArgs a) {
  const int h = blockIdx.x, t = blockIdx.y, layer = blockIdx.z;
  const int tid = threadIdx.x;
  const size_t base = ((size_t)layer * a.T + t) * a.n_slots;
  __shared__ float fac[64];
  __shared__ float s_inv;
  // all slot loads in flight at once (at most kMaxSlots slots), before the weights are known
  uint2 o[kMaxSlots];
#pragma unroll
  for (int s = 0; s < kMaxSlots; ++s)
    if (s < a.n_slots) o[s] = *reinterpret_cast<const uint2*>(a.part_o + ((base + s) * kHeads + h) * kDim + 4 * tid);
  if (tid < 64) {
    // one lane per slot (n_slots <= 64): max, then weighted sum, by wave reductions
    const bool has = tid < a.n_slots;
    const float ms = has ? a.part_ml[((base + tid) * kHeads + h) * 2] : -INFINITY;
    const float ls = has ? a.part_ml[((base + tid) * kHeads + h) * 2 + 1] : 0.f;
    float M = wave_max_dpp(ms);
    float sk = -INFINITY;
    if (a.sink) {
      sk = a.sink[(size_t)layer * kHeads + h] * kLog2e;
      M = fmaxf(M, sk);
    }
    const float f = (M == -INFINITY || ms == -INFINITY) ? 0.f : exp2f(ms - M);
    float den = wave_sum_dpp(ls * f);
    if (a.sink && M != -INFINITY) den += exp2f(sk - M);
    if (has) fac[tid] = f;
    if (tid == 0) {
      s_inv = (M == -INFINITY || den == 0.f) ? 0.f : 1.f / den;
      if (a.lse) a.lse[((size_t)layer * a.T + t) * kHeads + h] = (M == -INFINITY) ? -INFINITY : (M + log2f(den)) * kLn2;
    }
  }
  __syncthreads();
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < kMaxSlots; ++s)
    if (s < a.n_slots && fac[s] != 0.f) {
      const floatx4 v = {bf16lo(o[s].x), bf16hi(o[s].x), bf16lo(o[s].y), bf16hi(o[s].y)};
      acc += v * fac[s];
    }
  const float iv = s_inv;
  uint16_t* op = a.out + (((size_t)layer * a.T + t) * kHeads + h) * kDim + 4 * tid;
  float v[4] = {acc[0] * iv, acc[1] * iv, acc[2] * iv, acc[3] * iv};
  if (tid >= 112 && a.rope_pos) {  // channels 448..511: pairs (v0, v1), (v2, v3)
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      float c, sn;
      rope_cs(a, t, 2 * (tid - 112) + p, &c, &sn);
      const float x = v[2 * p], y = v[2 * p + 1];
      v[2 * p] = x * c - y * sn;
      v[2 * p + 1] = x * sn + y * c;
    }
  }
  const uint32_t w0 = pack_bf16x2_rne(v[0], v[1]);
  const uint32_t w1 = pack_bf16x2_rne(v[2], v[3]);
  *reinterpret_cast<uint2*>(op) = make_uint2(w0, w1);
}

struct AttendPlan {
  int n_main, n_swa, cpw, n_items, n_slots;
};

static AttendPlan attend_plan(int32_t T, int32_t k, int32_t window, int32_t L) {
  AttendPlan p;
  p.n_main = (k + kChunk - 1) / kChunk;
  p.n_swa = (window + kChunk - 1) / kChunk;
  const int n_chunks = p.n_main + p.n_swa;
  if (L == 1) {
    // enough work items to cover the GPU (~1024 blocks), merged back by the combine
    int64_t want = (1024 + T - 1) / T;
    if (want > n_chunks) want = n_chunks;
    if (want < 1) want = 1;
    p.cpw = (int)((n_chunks + want - 1) / want);
    p.n_items = (n_chunks + p.cpw - 1) / p.cpw;
    p.n_slots = p.n_items;
  } else {
    p.cpw = 1;
    p.n_items = p.n_main + L * p.n_swa;
    p.n_slots = n_chunks;
  }
  return p;
}

static size_t attend_ws_bytes(int32_t T, const AttendPlan& p, int32_t L) {
  if (p.n_items == 1 && L == 1) return 0;
  const size_t slots = (size_t)L * T * p.n_slots;
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
  const AttendPlan p = attend_plan(T, k, window, L);
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
  a.n_slots = p.n_slots;
  a.out = (uint16_t*)out;
  a.lse = lse;
  const size_t slots = (size_t)L * T * p.n_slots;
  a.part_o = need ? (uint16_t*)workspace : nullptr;
  a.part_ml = need ? (float*)((char*)workspace + align_up(slots * kHeads * kDim * sizeof(uint16_t), 256)) : nullptr;
  hipStream_t st = (hipStream_t)hip_stream;
  (void)hipGetLastError();
  // small batches: one wave per block and four blocks per work item (16 heads
  // each), so that the work and the partial writes spread over four times the CUs
  const bool one = (int64_t)p.n_items * T * 4 <= 4096;
  const dim3 grid(p.n_items, T, one ? 4 : 1), block(one ? 64 : kAttnThreads);
  const int fmt = 2 * o.kv_format + o.swa_format;
#define CSA2_ATTEND(W, KVF, SWF) hipLaunchKernelGGL((attend_kernel<W, KVF, SWF>), grid, block, 0, st, a)
  if (one) {
    if (fmt == 0) CSA2_ATTEND(1, 0, 0);
    else if (fmt == 1) CSA2_ATTEND(1, 0, 1);
    else if (fmt == 2) CSA2_ATTEND(1, 1, 0);
    else CSA2_ATTEND(1, 1, 1);
  } else {
    if (fmt == 0) CSA2_ATTEND(4, 0, 0);
    else if (fmt == 1) CSA2_ATTEND(4, 0, 1);
    else if (fmt == 2) CSA2_ATTEND(4, 1, 0);
    else CSA2_ATTEND(4, 1, 1);
  }
#undef CSA2_ATTEND
  if (need) hipLaunchKernelGGL(attend_combine_kernel, dim3(kHeads, T, L), dim3(128), 0, st, a);
  if (hipGetLastError() != hipSuccess) return CSA2_ERR_LAUNCH;
  return CSA2_OK;
}

}  // namespace csa2

using namespace csa2;

extern "C" size_t csa2_attend_workspace_bytes(int32_t T, int32_t k, int32_t window, int32_t n_layers) {
  if (T < 1 || k != kTopK || window < 1 || window > CSA2_MAX_WINDOW || n_layers < 1 || n_layers > CSA2_MAX_LAYERS)
    return 0;
  const AttendPlan p = attend_plan(T, k, window, n_layers);
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
