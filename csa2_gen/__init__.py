"""Seeded synthetic inputs for CSA2 — shared by the HIP path's tests/bench and the oracle.

This module holds no part of the method's arithmetic: it only draws numbers
and packs them into the storage formats the hot path reads.

Every element is a pure function of (seed, stream, flat element index), so any
slice of any tensor can be regenerated on the CPU or on the GPU with identical
bytes (all steps are integer operations plus exact float ops):

  * 64-bit counter hash: SplitMix64 (Steele, Lea, Flood, "Fast splittable
    pseudorandom number generators", OOPSLA 2014) applied to
    seed * A + stream * B + index.
  * N(0,1) in bf16: the top 16 hash bits pick one of 65536 equiprobable bins;
    the bin's value is the standard-normal quantile at its midpoint, rounded to
    float32 and then to bf16 (round to nearest even).
  * U(0,1) in fp32: the top 24 hash bits times 2^-24.
  * MXFP4 (OCP Microscaling E2M1 + E8M0, 32 elements per scale): shared scale
    2^(floor(log2 amax) - 2), elements rounded to nearest E2M1 value with ties to
    the even code, saturating at 6; an all-zero block gets scale code 127.  This
    is the KV *write* side (upstream of the hot path), used here only to make
    the cache bytes the path consumes.
"""
from __future__ import annotations

import math
import statistics
from dataclasses import dataclass, field

import numpy as np
import torch

MASK64 = (1 << 64) - 1
_A = 0xD1B54A32D192ED03
_B = 0xABC98388FB8FAC03
_GOLDEN = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB

# tensor streams
ST_QIDX, ST_W, ST_KIDX, ST_KV, ST_Q, ST_SWA = 1, 2, 3, 4, 16, 64

IDX_HEADS, IDX_DIM, HEADS, DIM, MX_BLOCK = 32, 128, 64, 512, 32


def _s64(v: int) -> int:
    v &= MASK64
    return v - (1 << 64) if v >= (1 << 63) else v


def _lsr(x: torch.Tensor, k: int) -> torch.Tensor:
    return (x >> k) & ((1 << (64 - k)) - 1)


def hash64(seed: int, stream: int, idx: torch.Tensor) -> torch.Tensor:
    """SplitMix64 of (seed*A + stream*B + idx) as int64 (two's complement bits)."""
    x = idx.to(torch.int64) + _s64(seed * _A + stream * _B + _GOLDEN)
    x = (x ^ _lsr(x, 30)) * _s64(_M1)
    x = (x ^ _lsr(x, 27)) * _s64(_M2)
    return x ^ _lsr(x, 31)


def hash64_ref(seed: int, stream: int, i: int) -> int:
    """Pure-Python reference of hash64 for one element (unsigned result)."""
    x = (i + seed * _A + stream * _B + _GOLDEN) & MASK64
    x = ((x ^ (x >> 30)) * _M1) & MASK64
    x = ((x ^ (x >> 27)) * _M2) & MASK64
    return x ^ (x >> 31)


def _f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    u = np.asarray(a, np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


_NORMAL_TABLE = None


def normal_table() -> np.ndarray:
    """65536 bf16 bit patterns: N(0,1) quantiles at bin midpoints (uint16)."""
    global _NORMAL_TABLE
    if _NORMAL_TABLE is None:
        nd = statistics.NormalDist()
        vals = np.array([nd.inv_cdf((i + 0.5) / 65536.0) for i in range(65536)], np.float64)
        _NORMAL_TABLE = _f32_to_bf16_bits(vals.astype(np.float32))
    return _NORMAL_TABLE


_TABLE_CACHE: dict = {}


def _table_on(device) -> torch.Tensor:
    key = str(device)
    if key not in _TABLE_CACHE:
        t = torch.from_numpy(normal_table().astype(np.int32)).to(torch.int16)
        _TABLE_CACHE[key] = t.to(device)
    return _TABLE_CACHE[key]


def normal_bf16(seed: int, stream: int, start: int, count: int, device="cpu") -> torch.Tensor:
    """Elements [start, start+count) of a stream as bf16 bit patterns (int16)."""
    idx = torch.arange(start, start + count, dtype=torch.int64, device=device)
    h = hash64(seed, stream, idx)
    bins = _lsr(h, 48)
    return _table_on(device)[bins]


def normal_bf16_rows(seed: int, stream: int, rows: torch.Tensor, row_len: int) -> torch.Tensor:
    """Selected rows (int64 row ids) of a [*, row_len] stream -> int16 [len(rows)][row_len]."""
    dev = rows.device
    idx = rows.to(torch.int64)[:, None] * row_len + torch.arange(row_len, device=dev, dtype=torch.int64)[None, :]
    h = hash64(seed, stream, idx)
    return _table_on(dev)[_lsr(h, 48)]


def uniform_f32(seed: int, stream: int, start: int, count: int, device="cpu") -> torch.Tensor:
    idx = torch.arange(start, start + count, dtype=torch.int64, device=device)
    h = hash64(seed, stream, idx)
    return _lsr(h, 40).to(torch.float32) * (2.0 ** -24)


def bf16_bits_to_float(b: torch.Tensor) -> torch.Tensor:
    return (b.to(torch.int32) << 16).view(torch.float32)


def mxfp4_quantize(x_bits: torch.Tensor):
    """bf16 bits int16 [R][D] -> (codes uint8 [R][D/2], scales uint8 [R][D/32])."""
    R, D = x_bits.shape
    x = bf16_bits_to_float(x_bits).view(R, D // MX_BLOCK, MX_BLOCK)
    amax = x.abs().amax(dim=2)
    _, ex = torch.frexp(amax)                      # amax = m * 2^ex, m in [0.5, 1)
    shared = torch.where(amax > 0, ex - 1 - 2, torch.zeros_like(ex))   # floor(log2 amax) - emax(E2M1)
    scale_code = (shared + 127).clamp(0, 254).to(torch.uint8)
    # exact power-of-two scaling in fp64: 2^(-shared) built from its bit pattern
    pow2 = ((1023 - shared.to(torch.int64)) << 52).view(torch.float64)
    scaled = x.to(torch.float64) * pow2[:, :, None]
    a = scaled.abs()
    mag = ((a > 0.25).to(torch.int32) + (a >= 0.75).to(torch.int32) + (a > 1.25).to(torch.int32)
           + (a >= 1.75).to(torch.int32) + (a > 2.5).to(torch.int32) + (a >= 3.5).to(torch.int32)
           + (a > 5.0).to(torch.int32))
    code = mag | ((scaled < 0).to(torch.int32) << 3)
    code = code.view(R, D // 2, 2)
    packed = (code[:, :, 0] | (code[:, :, 1] << 4)).to(torch.uint8)
    return packed, scale_code.view(R, D // MX_BLOCK)


# ---------------------------------------------------------------- workloads

@dataclass
class Case:
    """One CSA2 workload: all tensors for a Full layer (+ optional Reuse layers)."""
    name: str
    B: int
    N: int
    q_per_seq: int
    ratio: int
    S: int
    window: int
    k: int
    n_layers: int           # 1 Full + (n_layers - 1) Reuse layers
    seed: int
    softmax_scale: float
    q_pos: torch.Tensor = None      # int32 [T]
    swa_end: torch.Tensor = None    # int32 [T]
    q_idx: torch.Tensor = None      # bf16 bits int16 [T][32][128]
    w_idx: torch.Tensor = None      # float32 [T][32]
    k_idx: torch.Tensor = None      # int16 [B][N][128]
    kv_codes: torch.Tensor = None   # uint8 [B][N][256]
    kv_scales: torch.Tensor = None  # uint8 [B][N][16]
    q: torch.Tensor = None          # int16 [L][T][64][512]
    swa: torch.Tensor = None        # int16 [L][B][S][512]
    extra: dict = field(default_factory=dict)

    @property
    def T(self) -> int:
        return self.B * self.q_per_seq


def make_case(name, B, N, q_per_seq=1, ratio=1, prefix=None, window=128, k=512, n_layers=1,
              seed=0, device="cpu", with_kv=True, chunk_rows=1 << 16) -> Case:
    """Build a seeded workload.

    Decode (prefix None): query t is the latest token of its sequence, position
    ratio*N - 1, so all N entries are visible; the SWA tensor holds that token's
    `window` most recent tokens (S = window rows, window end = S).
    Prefill (prefix P, B=1): queries are tokens P .. P+T-1; N must equal
    (P+T)//ratio; the SWA tensor holds tokens P-window+1 .. P+T-1
    (S = T + window - 1) and query t's window ends after row t + window - 1.
    """
    T = B * q_per_seq
    c = Case(name=name, B=B, N=N, q_per_seq=q_per_seq, ratio=ratio, S=0, window=window, k=k,
             n_layers=n_layers, seed=seed, softmax_scale=1.0 / math.sqrt(DIM))
    if prefix is None:
        c.q_pos = torch.full((T,), ratio * N - 1, dtype=torch.int32)
        c.S = window
        c.swa_end = torch.full((T,), window, dtype=torch.int32)
    else:
        assert B == 1 and (prefix + T) // ratio == N
        c.q_pos = torch.arange(prefix, prefix + T, dtype=torch.int32)
        c.S = T + window - 1
        c.swa_end = torch.arange(window, window + T, dtype=torch.int32)
    c.q_pos, c.swa_end = c.q_pos.to(device), c.swa_end.to(device)
    c.q_idx = normal_bf16(seed, ST_QIDX, 0, T * IDX_HEADS * IDX_DIM, device).view(T, IDX_HEADS, IDX_DIM)
    c.w_idx = uniform_f32(seed, ST_W, 0, T * IDX_HEADS, device).view(T, IDX_HEADS)
    c.k_idx = torch.empty((B, N, IDX_DIM), dtype=torch.int16, device=device)
    flat_k = c.k_idx.view(-1)
    total = B * N * IDX_DIM
    step = chunk_rows * IDX_DIM * 4
    for s0 in range(0, total, step):
        n = min(step, total - s0)
        flat_k[s0:s0 + n] = normal_bf16(seed, ST_KIDX, s0, n, device)
    if with_kv:
        c.kv_codes = torch.empty((B, N, DIM // 2), dtype=torch.uint8, device=device)
        c.kv_scales = torch.empty((B, N, DIM // MX_BLOCK), dtype=torch.uint8, device=device)
        rows = B * N
        fc, fs = c.kv_codes.view(rows, -1), c.kv_scales.view(rows, -1)
        for r0 in range(0, rows, chunk_rows):
            n = min(chunk_rows, rows - r0)
            x = normal_bf16(seed, ST_KV, r0 * DIM, n * DIM, device).view(n, DIM)
            fc[r0:r0 + n], fs[r0:r0 + n] = mxfp4_quantize(x)
    c.q = torch.stack([normal_bf16(seed, ST_Q + l, 0, T * HEADS * DIM, device).view(T, HEADS, DIM)
                       for l in range(n_layers)])
    c.swa = torch.stack([normal_bf16(seed, ST_SWA + l, 0, B * c.S * DIM, device).view(B, c.S, DIM)
                         for l in range(n_layers)])
    return c


def e4m3_encode(v: torch.Tensor) -> torch.Tensor:
    """Nearest OCP E4M3 code of float64 values (ties to the even code), saturating at 448."""
    a = v.abs().clamp(max=448.0)
    sign = (v < 0).to(torch.int32) << 7
    _, ex = torch.frexp(a)                         # a = f * 2^ex, f in [0.5, 1)
    e = (ex - 1).clamp(min=-6)                     # unbiased exponent, subnormals share 2^-6
    step = torch.ldexp(torch.ones_like(a), (e - 3).to(torch.int32))   # spacing of codes at that exponent
    q = a / step                                   # exact: step is a power of two
    r = torch.floor(q)
    frac = q - r
    r = r + ((frac > 0.5) | ((frac == 0.5) & (r.remainder(2) == 1))).to(r.dtype)
    # r counts steps: subnormal codes are r (0..8), normal codes (e + 7) * 8 + (r - 8)
    normal = e > -6
    code = torch.where(normal, (e + 7) * 8 + (r.to(torch.int32) - 8), r.to(torch.int32))
    code = torch.where(a == 0, torch.zeros_like(code), code).clamp(max=0x7E)
    return (code | sign).to(torch.uint8)


def e4m3_decode(code: torch.Tensor) -> torch.Tensor:
    c = code.to(torch.int32)
    e, m = (c >> 3) & 15, c & 7
    mag = torch.where(e == 0, m.to(torch.float64) * 2.0 ** -9,
                      torch.ldexp(8.0 + m.to(torch.float64), (e - 10).to(torch.int32)))
    return torch.where((c & 0x80) != 0, -mag, mag)


def _e2m1_codes(scaled: torch.Tensor) -> torch.Tensor:
    """RNE to E2M1 (ties to the even code), saturating at 6; scaled float64 -> int32 codes."""
    a = scaled.abs()
    mag = ((a > 0.25).to(torch.int32) + (a >= 0.75).to(torch.int32) + (a > 1.25).to(torch.int32)
           + (a >= 1.75).to(torch.int32) + (a > 2.5).to(torch.int32) + (a >= 3.5).to(torch.int32)
           + (a > 5.0).to(torch.int32))
    return mag | ((scaled < 0).to(torch.int32) << 3)


def e4m3_16_quantize(x_bits: torch.Tensor):
    """bf16 bits int16 [R][D] -> (E2M1 codes uint8 [R][D/2], E4M3 scales uint8 [R][D/16]).
    Per block of 16: scale = E4M3 nearest to amax / 6, elements x / scale rounded to E2M1."""
    R, D = x_bits.shape
    x = bf16_bits_to_float(x_bits).to(torch.float64).view(R, D // 16, 16)
    amax = x.abs().amax(dim=2)
    sc_code = e4m3_encode(amax / 6.0)
    sc = e4m3_decode(sc_code)
    scaled = torch.where(sc[:, :, None] > 0, x / torch.where(sc > 0, sc, 1.0)[:, :, None], torch.zeros_like(x))
    code = _e2m1_codes(scaled).view(R, D // 2, 2)
    packed = (code[:, :, 0] | (code[:, :, 1] << 4)).to(torch.uint8)
    return packed, sc_code.view(R, D // 16)


def fp8_window_quantize(x_bits: torch.Tensor):
    """bf16 bits int16 [R][512] -> (E4M3 uint8 [R][448], bf16 bits int16 [R][64], E8M0 uint8 [R][8]).
    Channels 0..447 in blocks of 64: shared exponent floor(log2 amax) - 8 (the E4M3 maximum
    exponent), elements rounded to E4M3 (saturating at 448); channels 448..511 kept as bf16."""
    R = x_bits.shape[0]
    x = bf16_bits_to_float(x_bits[:, :448]).to(torch.float64).view(R, 7, 64)
    amax = x.abs().amax(dim=2)
    _, ex = torch.frexp(amax)
    shared = torch.where(amax > 0, ex - 1 - 8, torch.zeros_like(ex))
    scale_code = (shared + 127).clamp(0, 254)
    pow2 = ((1023 - (scale_code.to(torch.int64) - 127)) << 52).view(torch.float64)
    fp8 = e4m3_encode(x * pow2[:, :, None]).view(R, 448)
    scales = torch.zeros((R, 8), dtype=torch.uint8, device=x_bits.device)
    scales[:, :7] = scale_code.to(torch.uint8)
    return fp8, x_bits[:, 448:].contiguous(), scales


def kv_e4m3_16(c: "Case", chunk_rows: int = 1 << 16):
    """The case's main KV (the same seeded bf16 rows its MXFP4 cache quantises) in the E2M1 +
    E4M3/16 format -> (codes uint8 [B][N][256], scales uint8 [B][N][32])."""
    rows = c.B * c.N
    dev = c.kv_codes.device
    codes = torch.empty((rows, DIM // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((rows, DIM // 16), dtype=torch.uint8, device=dev)
    for r0 in range(0, rows, chunk_rows):
        n = min(chunk_rows, rows - r0)
        x = normal_bf16(c.seed, ST_KV, r0 * DIM, n * DIM, dev).view(n, DIM)
        codes[r0:r0 + n], scales[r0:r0 + n] = e4m3_16_quantize(x)
    return codes.view(c.B, c.N, DIM // 2), scales.view(c.B, c.N, DIM // 16)


def window_fp8(c: "Case"):
    """The case's window rows (every layer) in the FP8 layout -> (fp8 [L][B][S][448],
    rope bf16 bits [L][B][S][64], scales [L][B][S][8])."""
    L, B, S = c.swa.shape[0], c.swa.shape[1], c.swa.shape[2]
    f, r, s = fp8_window_quantize(c.swa.reshape(L * B * S, DIM))
    return f.view(L, B, S, 448), r.view(L, B, S, 64), s.view(L, B, S, 8)


def mx_indexer(c: "Case", chunk_rows: int = 1 << 16):
    """MXFP4 indexer operands quantised from the case's bf16 indexer queries and keys
    -> (q_codes uint8 [T][32][64], q_scales uint8 [T][32][4], k_codes uint8 [B][N][64],
    k_scales uint8 [B][N][4]), on the case's device."""
    T, B, N = c.T, c.B, c.N
    qc, qs = mxfp4_quantize(c.q_idx.reshape(T * IDX_HEADS, IDX_DIM))
    kc = torch.empty((B * N, IDX_DIM // 2), dtype=torch.uint8, device=c.k_idx.device)
    ks = torch.empty((B * N, IDX_DIM // MX_BLOCK), dtype=torch.uint8, device=c.k_idx.device)
    flat = c.k_idx.reshape(B * N, IDX_DIM)
    for r0 in range(0, B * N, chunk_rows):
        r1 = min(B * N, r0 + chunk_rows)
        kc[r0:r1], ks[r0:r1] = mxfp4_quantize(flat[r0:r1])
    return (qc.view(T, IDX_HEADS, IDX_DIM // 2), qs.view(T, IDX_HEADS, IDX_DIM // MX_BLOCK),
            kc.view(B, N, IDX_DIM // 2), ks.view(B, N, IDX_DIM // MX_BLOCK))


def kv_rows(seed: int, rows: torch.Tensor):
    """Regenerate selected flat KV rows (b*N + s) -> (codes, scales)."""
    x = normal_bf16_rows(seed, ST_KV, rows, DIM)
    return mxfp4_quantize(x)


# Streams of the KV-write inputs (hidden states, projection weights, positions).
ST_H, ST_WKV, ST_WZ, ST_WIK, ST_POS = 200, 201, 202, 203, 204


def _scaled_normal_bf16(seed: int, stream: int, count: int, exp2: int, device) -> torch.Tensor:
    """N(0,1) bf16 bits times 2^exp2 (exact: only the exponent changes)."""
    f = bf16_bits_to_float(normal_bf16(seed, stream, 0, count, device)) * (2.0 ** exp2)
    return (f.view(torch.int32) >> 16).to(torch.int16)


def kv_write_inputs(seed: int, n_ent: int, m: int, d: int, device="cpu", max_pos: int = 1 << 20):
    """Inputs of the KV write for n_ent entries of m tokens with hidden size d (bf16 bits as int16):
    h [n_ent*m][d] ~ N(0,1); w_kv, w_z [512][d] ~ N(0,1) * 2^-6 (w_z None when m == 1);
    w_ik [128][512] ~ N(0,1) * 2^-4; pos int32 [n_ent] uniform in [0, max_pos).  The weight
    scales keep the pooled entries and the indexer keys of order one for d near 5120."""
    h = normal_bf16(seed, ST_H, 0, n_ent * m * d, device).view(n_ent * m, d)
    w_kv = _scaled_normal_bf16(seed, ST_WKV, DIM * d, -6, device).view(DIM, d)
    w_z = _scaled_normal_bf16(seed, ST_WZ, DIM * d, -6, device).view(DIM, d) if m > 1 else None
    w_ik = _scaled_normal_bf16(seed, ST_WIK, IDX_DIM * DIM, -4, device).view(IDX_DIM, DIM)
    pos = (uniform_f32(seed, ST_POS, 0, n_ent, device) * max_pos).to(torch.int32)
    return dict(h=h, w_kv=w_kv, w_z=w_z, w_ik=w_ik, pos=pos)


# Workloads named by what they are (batch, entries, mode).
CONFIGS = {
    "tiny_decode": dict(B=1, N=2048),
    "batched_decode": dict(B=64, N=131072),
    "reuse_group": dict(B=32, N=262144, n_layers=4),
    "causal_prefill": dict(B=1, N=34816, q_per_seq=4096, ratio=2, prefix=65536),
    "long_decode": dict(B=4, N=1048576),
}


def algorithmic_bytes_decode_query(N: int, k: int = 512, window: int = 128) -> int:
    """Bytes one decode query must move at minimum: indexer keys (256 B/entry),
    indexer q (8 KiB) and w (128 B), k FP4 rows (256 B codes + 16 B scales),
    the window's bf16 rows (1 KiB each), q (64 KiB), out (64 KiB), indices (4 B each)."""
    return 256 * N + 8192 + 128 + k * 272 + window * 1024 + 65536 + 65536 + 4 * k
