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
// Two kernels.
//  kvw_proj_kernel   C (and Z) on v_mfma_f32_16x16x32_bf16.  A wave owns 16
//                    tokens x 64 channels over a slice of the hidden
//                    dimension.  Many tokens (prefill): the 4 waves of a block
//                    take 4 token tiles of one channel chunk and share its
//                    weight rows through the caches.  Few tokens (decode): the
//                    hidden dimension is split over waves and blocks so that
//                    the weight stream (512 x d x 2 B per projection) is in
//                    flight on the whole GPU at once; per-slice sums go to the
//                    workspace.
//  kvw_finish_kernel one block per (16-token tile, 64-channel chunk): adds the
//                    slice sums, pools, rotates and quantises the chunk (64
//                    channels hold whole 16- and 32-channel scale blocks),
//                    and writes the chunk's share of indexer K.  The last of
//                    the 8 chunk blocks of a tile (an arrival counter, zeroed
//                    by the projection kernel) adds the 8 shares in chunk order
//                    and writes K.  Every sum has a fixed order: results do not
//                    depend on scheduling.
#include "mxfp4.h"

namespace csa2 {

constexpr int kKvwTok = 16;                     // tokens per tile (MFMA rows)
constexpr int kKvwChunk = 64;                   // channels per chunk
constexpr int kKvwChunks = kDim / kKvwChunk;    // 8
constexpr int kKvwThreads = 256;                // projection block: 4 waves
constexpr int kKvwFinThreads = 1024;            // finish block: 16 waves, one token each
constexpr int kKvwMinSlice = 128;               // smallest hidden-dimension slice per wave
constexpr int kKvwWantWaves = 1024;             // projection waves aimed at for few tokens
constexpr int kKvwWikStride = kKvwChunk + 2;    // LDS row of W_ik (bf16): 33 words, rows on distinct banks

struct KvwPlan {
  int64_t n_tok;
  int tok_tiles;
  int tw;       // token tiles per projection block (4) or 1 (waves split the hidden dimension)
  int ksplit;   // hidden-dimension slices
  int kper;     // slice length (multiple of 32)
  int gx, gz;   // projection grid x and z (y = chunks)
  size_t off_z, off_kp, off_cnt, total;  // workspace layout (bytes)
};

static size_t kvw_round(size_t b) { return (b + 255) & ~(size_t)255; }

static KvwPlan kvw_plan(int32_t n_ent, int32_t m, int32_t d) {
  KvwPlan p;
  p.n_tok = (int64_t)n_ent * m;
  p.tok_tiles = (int)((p.n_tok + kKvwTok - 1) / kKvwTok);
  const int steps = d / 32;
  if (p.tok_tiles >= 64) {
    p.tw = 4;
    p.ksplit = 1;
    p.kper = d;
    p.gx = (p.tok_tiles + 3) / 4;
    p.gz = 1;
  } else {
    p.tw = 1;
    int64_t ks = (kKvwWantWaves + (int64_t)p.tok_tiles * kKvwChunks - 1) / ((int64_t)p.tok_tiles * kKvwChunks);
    const int kmax = d / kKvwMinSlice > 0 ? d / kKvwMinSlice : 1;
    if (ks > kmax) ks = kmax;
    if (ks < 1) ks = 1;
    p.kper = (int)((steps + ks - 1) / ks) * 32;
    p.ksplit = (d + p.kper - 1) / p.kper;  // every slice non-empty
    p.gx = p.tok_tiles;
    p.gz = (p.ksplit + 3) / 4;
  }
  const size_t part = (size_t)p.ksplit * p.n_tok * kDim * sizeof(float);
  p.off_z = kvw_round(part);
  p.off_kp = p.off_z + (m > 1 ? kvw_round(part) : 0);
  p.off_cnt = p.off_kp + kvw_round((size_t)kKvwChunks * n_ent * kIdxDim * sizeof(float));
  p.total = p.off_cnt + kvw_round((size_t)p.tok_tiles * sizeof(uint32_t));
  return p;
}

// part[split][token][channel]: the sum over slice `split` of h[token][k] * w[channel][k]
// (C), and at part + zoff the same for W_z.  Register i of lane l holds token 4(l/16) + i of
// the tile and channel l % 16 of each 16-channel group.
__global__ __launch_bounds__(kKvwThreads) void kvw_proj_kernel(const uint16_t* __restrict__ h,
                                                               const uint16_t* __restrict__ w_kv,
                                                               const uint16_t* __restrict__ w_z, int64_t n_tok,
                                                               int32_t d, int tok_tiles, int tw, int ksplit,
                                                               int kper, float* __restrict__ part, size_t zoff,
                                                               uint32_t* __restrict__ cnt) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tile = tw == 4 ? 4 * blockIdx.x + wave : blockIdx.x;
  const int split = tw == 4 ? blockIdx.z : 4 * blockIdx.z + wave;
  if (tile >= tok_tiles || split >= ksplit) return;
  if (blockIdx.y == 0 && split == 0 && lane == 0) cnt[tile] = 0u;  // arrival counter of the finish kernel
  const int r16 = lane & 15, g = lane >> 4;
  const int64_t tok = (int64_t)tile * kKvwTok + r16;
  const int ch0 = blockIdx.y * kKvwChunk + r16;
  const int k0 = split * kper;
  const int k1 = k0 + kper < d ? k0 + kper : d;
  // rows past n_tok read the last token again; their sums are not stored
  const uint16_t* hr = h + (size_t)(tok < n_tok ? tok : n_tok - 1) * d + 8 * g;
  const uint16_t* wr = w_kv + (size_t)ch0 * d + 8 * g;
  const uint16_t* zr = w_z ? w_z + (size_t)ch0 * d + 8 * g : nullptr;
  const size_t g16 = (size_t)16 * d;  // next 16-channel group
  floatx4 acc[4], accz[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    acc[c] = floatx4{0.f, 0.f, 0.f, 0.f};
    accz[c] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
  int k = k0;
  if (zr) {
    for (; k + 64 <= k1; k += 64) {
      uint4 a[2], b[2][4], z[2][4];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        a[u] = *reinterpret_cast<const uint4*>(hr + k + 32 * u);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          b[u][c] = *reinterpret_cast<const uint4*>(wr + c * g16 + k + 32 * u);
          z[u][c] = *reinterpret_cast<const uint4*>(zr + c * g16 + k + 32 * u);
        }
      }
      __builtin_amdgcn_sched_barrier(0);  // every load of the step group in flight before the first product
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[u]), as_bf16x8(b[u][c]), acc[c], 0, 0, 0);
          accz[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[u]), as_bf16x8(z[u][c]), accz[c], 0, 0, 0);
        }
    }
  } else {
    for (; k + 128 <= k1; k += 128) {
      uint4 a[4], b[4][4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        a[u] = *reinterpret_cast<const uint4*>(hr + k + 32 * u);
#pragma unroll
        for (int c = 0; c < 4; ++c) b[u][c] = *reinterpret_cast<const uint4*>(wr + c * g16 + k + 32 * u);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[u]), as_bf16x8(b[u][c]), acc[c], 0, 0, 0);
    }
  }
  for (; k < k1; k += 32) {
    const uint4 a = *reinterpret_cast<const uint4*>(hr + k);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint4 b = *reinterpret_cast<const uint4*>(wr + c * g16 + k);
      acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), acc[c], 0, 0, 0);
      if (zr) {
        const uint4 z = *reinterpret_cast<const uint4*>(zr + c * g16 + k);
        accz[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(z), accz[c], 0, 0, 0);
      }
    }
  }
  float* out = part + (size_t)split * n_tok * kDim;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t t = (int64_t)tile * kKvwTok + 4 * g + i;
    if (t < n_tok) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        out[(size_t)t * kDim + ch0 + 16 * c] = acc[c][i];
        if (zr) out[zoff + (size_t)t * kDim + ch0 + 16 * c] = accz[c][i];
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

__global__ __launch_bounds__(kKvwFinThreads) void kvw_finish_kernel(
    const float* __restrict__ part, size_t zoff, int ksplit, int64_t n_tok, int m,
    const uint16_t* __restrict__ w_ik, const int32_t* __restrict__ pos, double log2_base, int kv_format,
    uint8_t* __restrict__ kv_codes, uint8_t* __restrict__ kv_scales, int k_format, void* __restrict__ k_out,
    uint8_t* __restrict__ k_scales, float* __restrict__ kp, int32_t n_ent, uint32_t* __restrict__ cnt) {
  __shared__ float cz[2][kKvwTok][kKvwChunk];
  __shared__ float pre[kKvwTok][kKvwChunk];
  __shared__ uint16_t wik[kIdxDim * kKvwWikStride];
  __shared__ int is_last;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tile = blockIdx.x, chunk = blockIdx.y;
  const int64_t t0 = (int64_t)tile * kKvwTok;
  const int valid = n_tok - t0 < kKvwTok ? (int)(n_tok - t0) : kKvwTok;
  const int n_e = valid / m;            // entries of this tile (whole: m divides 16)
  const int e0 = tile * (kKvwTok / m);  // first entry of the tile
  {
    // W_ik columns of this chunk: row o, channels chunk*64 .. +63 -> LDS row o
    const int o = tid >> 3, seg = tid & 7;
    const uint4 w = *reinterpret_cast<const uint4*>(w_ik + (size_t)o * kDim + chunk * kKvwChunk + 8 * seg);
    uint32_t* dst = reinterpret_cast<uint32_t*>(wik + o * kKvwWikStride + 8 * seg);
    dst[0] = w.x;
    dst[1] = w.y;
    dst[2] = w.z;
    dst[3] = w.w;
  }
  // slice sums: wave = token of the tile, lane = channel of the chunk
  if (wave < valid) {
    const size_t off = (size_t)(t0 + wave) * kDim + chunk * kKvwChunk + lane;
    const size_t sstride = (size_t)n_tok * kDim;
    float c = 0.f, z = 0.f;
    int s = 0;
    for (; s + 8 <= ksplit; s += 8) {
      float v[8], u[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        v[i] = part[(size_t)(s + i) * sstride + off];
        u[i] = m > 1 ? part[zoff + (size_t)(s + i) * sstride + off] : 0.f;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        c += v[i];
        z += u[i];
      }
    }
    for (; s < ksplit; ++s) {
      c += part[(size_t)s * sstride + off];
      if (m > 1) z += part[zoff + (size_t)s * sstride + off];
    }
    cz[0][wave][lane] = c;
    cz[1][wave][lane] = z;
  }
  __syncthreads();
  // pooling, RoPE, quantisation: wave = entry of the tile, lane = channel
  if (wave < n_e) {
    const int e = e0 + wave;
    float v;
    if (m == 1) {
      v = cz[0][wave][lane];
    } else {
      float zmax = -INFINITY;
      for (int j = 0; j < m; ++j) zmax = fmaxf(zmax, cz[1][wave * m + j][lane]);
      float den = 0.f, num = 0.f;
      for (int j = 0; j < m; ++j) {
        const float p = expf(cz[1][wave * m + j][lane] - zmax);
        den += p;
        num += p * cz[0][wave * m + j][lane];
      }
      v = num / den;
    }
    pre[wave][lane] = v;
    if (chunk == kKvwChunks - 1) {
      // channel 448 + lane: pair j = lane / 2 with partner lane ^ 1
      const int j = lane >> 1;
      const double rev = (double)pos[e] * exp2(-log2_base * (j / 32.0)) * 0.15915494309189535;
      const float fr = (float)(rev - rint(rev));
      const float cs = __builtin_amdgcn_cosf(fr), sn = __builtin_amdgcn_sinf(fr);
      const float o = dpp_f32<kDppXor1>(v);
      v = (lane & 1) ? o * sn + v * cs : v * cs - o * sn;
    }
    uint32_t sc;
    const size_t cb = (size_t)e * (kDim / 2) + chunk * (kKvwChunk / 2) + (lane >> 1);
    if (kv_format == CSA2_KV_MXFP4) {
      const uint32_t byte = mx_quant_lane(v, &sc);
      if (!(lane & 1)) kv_codes[cb] = (uint8_t)byte;
      if (!(lane & 31)) kv_scales[(size_t)e * (kDim / 32) + chunk * 2 + (lane >> 5)] = (uint8_t)sc;
    } else {
      const uint32_t byte = e4m3_quant_lane(v, &sc);
      if (!(lane & 1)) kv_codes[cb] = (uint8_t)byte;
      if (!(lane & 15)) kv_scales[(size_t)e * (kDim / 16) + chunk * 4 + (lane >> 4)] = (uint8_t)sc;
    }
  }
  __syncthreads();
  // this chunk's share of indexer K: thread (o, g) for entries g, g + 8
  {
    const int o = tid & (kIdxDim - 1), g = tid >> 7;
    const uint32_t* wr = reinterpret_cast<const uint32_t*>(wik + o * kKvwWikStride);
    for (int el = g; el < n_e; el += 8) {
      float acc = 0.f;
#pragma unroll 8
      for (int c2 = 0; c2 < kKvwChunk / 2; ++c2) {
        const uint32_t w = wr[c2];
        acc = fmaf(pre[el][2 * c2], bf16lo(w), acc);
        acc = fmaf(pre[el][2 * c2 + 1], bf16hi(w), acc);
      }
      kp[((size_t)chunk * n_ent + e0 + el) * kIdxDim + o] = acc;
    }
  }
  // the last chunk block of the tile adds the shares in chunk order
  __threadfence();
  __syncthreads();
  if (tid == 0) is_last = atomicAdd(&cnt[tile], 1u) == kKvwChunks - 1;
  __syncthreads();
  if (!is_last) return;
  __threadfence();
  const int o = tid & (kIdxDim - 1), g = tid >> 7;
  for (int el = g; el < n_e; el += 8) {  // uniform per wave: a wave holds 64 outputs of one entry
    const int e = e0 + el;
    float kv = 0.f;
#pragma unroll
    for (int c = 0; c < kKvwChunks; ++c) kv += __builtin_nontemporal_load(&kp[((size_t)c * n_ent + e) * kIdxDim + o]);
    if (k_format == CSA2_K_BF16) {
      reinterpret_cast<uint16_t*>(k_out)[(size_t)e * kIdxDim + o] = (uint16_t)f32_to_bf16_rne(kv);
    } else {
      uint32_t sc;
      const uint32_t byte = mx_quant_lane(kv, &sc);
      if (!(lane & 1)) reinterpret_cast<uint8_t*>(k_out)[(size_t)e * kMxRowBytes + (o >> 1)] = (uint8_t)byte;
      if (!(lane & 31)) k_scales[(size_t)e * kMxScales + (o >> 5)] = (uint8_t)sc;
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
  char* ws = (char*)workspace;
  float* part = (float*)ws;
  const size_t zoff = p.off_z / sizeof(float);
  float* kp = (float*)(ws + p.off_kp);
  uint32_t* cnt = (uint32_t*)(ws + p.off_cnt);
  (void)hipGetLastError();
  hipLaunchKernelGGL(kvw_proj_kernel, dim3(p.gx, kKvwChunks, p.gz), dim3(kKvwThreads), 0, st, (const uint16_t*)h,
                     (const uint16_t*)w_kv, m > 1 ? (const uint16_t*)w_z : nullptr, p.n_tok, d, p.tok_tiles, p.tw,
                     p.ksplit, p.kper, part, zoff, cnt);
  hipLaunchKernelGGL(kvw_finish_kernel, dim3(p.tok_tiles, kKvwChunks), dim3(kKvwFinThreads), 0, st,
                     (const float*)part, zoff, p.ksplit, p.n_tok, m, (const uint16_t*)w_ik, pos,
                     log2((double)rope_base), kv_format, kv_codes, kv_scales, k_format, k_out, k_scales, kp, n_ent,
                     cnt);
  if (hipGetLastError() != hipSuccess) return CSA2_ERR_LAUNCH;
  return CSA2_OK;
}
