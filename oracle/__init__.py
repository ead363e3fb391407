"""CSA2 CPU oracle — TEST INFRASTRUCTURE ONLY.

Plain fp64 C implementation of the CSA2 hot path (csa2_oracle.c) behind a thin
ctypes wrapper over numpy arrays.  Only the tests, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import this package; the product
library never does.  It shares no code with the HIP library.

Functions follow the DeepSeek-V4.1-Flash report (sec. 2.3, 2.3.1, 2.3.2, 2.4.4,
3.2.2, 4.2.1) and the gzher.com reading of DeepSeek-V4 (sec. 4.1, 4.3); the
C source cites the passage for each step.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "csa2_oracle.c")
LIB_PLAIN = os.path.join(HERE, "libcsa2_oracle.so")
# AddressSanitizer + UndefinedBehaviorSanitizer build (clang, its runtime preloaded into the
# test process): CSA2_SANITIZE=1 selects it, for the oracle and the HIP library's host code alike
LIB_SAN = os.path.join(HERE, "libcsa2_oracle_san.so")
SANITIZE = os.environ.get("CSA2_SANITIZE", "") not in ("", "0")
LIB = LIB_SAN if SANITIZE else LIB_PLAIN
CLANG = "/opt/rocm/llvm/bin/clang"

IDX_HEADS, IDX_DIM, HEADS, DIM = 32, 128, 64, 512

_lib = None


def build(force: bool = True, sanitize: bool = None) -> str:
    """Compile the oracle with gcc (fp64, no fast-math, no contraction); with sanitize (default:
    CSA2_SANITIZE set) the same flags under clang with AddressSanitizer and UndefinedBehavior-
    Sanitizer (any report aborts)."""
    san = SANITIZE if sanitize is None else sanitize
    out = LIB_SAN if san else LIB_PLAIN
    if force or not os.path.exists(out):
        common = ["-O2", "-mfma", "-ffp-contract=off", "-fno-fast-math", "-shared", "-fPIC", "-std=c11",
                  "-Wall", "-Wextra", "-Werror"]
        if san:
            cmd = [CLANG, *common, "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                   "-fno-sanitize-recover=all", "-fopenmp", SRC, "-o", out + ".tmp", "-lm"]
        else:
            cmd = ["gcc", *common, "-fopenmp", SRC, "-o", out + ".tmp", "-lm"]
        subprocess.check_call(cmd)
        os.replace(out + ".tmp", out)
    return out


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        L = ctypes.CDLL(LIB)
        vp, i32, i64, dbl = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        L.csa2o_max_threads.argtypes, L.csa2o_max_threads.restype = [], i32
        L.csa2o_set_threads.argtypes, L.csa2o_set_threads.restype = [i32], i32
        L.csa2o_e2m1.argtypes, L.csa2o_e2m1.restype = [ctypes.c_uint32], dbl
        L.csa2o_e8m0.argtypes, L.csa2o_e8m0.restype = [ctypes.c_uint32], dbl
        L.csa2o_dequant_row.argtypes, L.csa2o_dequant_row.restype = [vp, vp, i32, vp], None
        L.csa2o_n_visible.argtypes, L.csa2o_n_visible.restype = [i64, i32, i64], i64
        L.csa2o_index_score.argtypes, L.csa2o_index_score.restype = [vp, vp, vp], dbl
        L.csa2o_index.argtypes = [vp, vp, vp, vp, i32, i32, i32, i64, vp]
        L.csa2o_index_score_deq.argtypes, L.csa2o_index_score_deq.restype = [vp, vp, vp], dbl
        L.csa2o_index_mx.argtypes, L.csa2o_index_mx.restype = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i64, vp], None
        L.csa2o_index.restype = None
        L.csa2o_topk_row.argtypes, L.csa2o_topk_row.restype = [vp, i64, i32, vp], i32
        L.csa2o_topk.argtypes, L.csa2o_topk.restype = [vp, vp, i32, i32, i64, i32, vp], None
        L.csa2o_topk_bf16.argtypes, L.csa2o_topk_bf16.restype = [vp, vp, i32, i32, i64, i32, vp], None
        L.csa2o_bf16_round.argtypes, L.csa2o_bf16_round.restype = [dbl], dbl
        L.csa2o_attend.argtypes = [vp, vp, vp, vp, vp, vp, vp, dbl, i32, i32, i64, i32, i32, i32, vp, vp]
        L.csa2o_attend_ex.argtypes = [vp, vp, vp, i32, vp, vp, vp, vp, vp, i32, vp, vp, dbl, i32, i32, i64, i32, i32,
                                      i32, vp, dbl, vp, vp]
        L.csa2o_attend_ex.restype = None
        L.csa2o_e4m3.argtypes, L.csa2o_e4m3.restype = [ctypes.c_uint32], dbl
        L.csa2o_dequant_row_e4m3.argtypes, L.csa2o_dequant_row_e4m3.restype = [vp, vp, i32, vp], None
        L.csa2o_dequant_swa_fp8_row.argtypes, L.csa2o_dequant_swa_fp8_row.restype = [vp, vp, vp, vp], None
        L.csa2o_rope_rotate.argtypes, L.csa2o_rope_rotate.restype = [vp, dbl, dbl], None
        L.csa2o_e2m1_encode.argtypes, L.csa2o_e2m1_encode.restype = [dbl], ctypes.c_uint32
        L.csa2o_e4m3_encode.argtypes, L.csa2o_e4m3_encode.restype = [dbl], ctypes.c_uint32
        L.csa2o_quantize_mx_block.argtypes, L.csa2o_quantize_mx_block.restype = [vp, vp, vp], None
        L.csa2o_quantize_e4m3_block.argtypes, L.csa2o_quantize_e4m3_block.restype = [vp, vp, vp], None
        L.csa2o_kv_write.argtypes = [vp, vp, vp, vp, i32, i32, i32, vp, dbl, i32, vp, vp, vp, vp, vp]
        L.csa2o_kv_write.restype = None
        L.csa2o_attend.restype = None
        L.csa2o_hsi_pool_row.argtypes, L.csa2o_hsi_pool_row.restype = [vp, i64, i32, i32, vp], i32
        L.csa2o_hsi_pool.argtypes, L.csa2o_hsi_pool.restype = [vp, vp, i32, i32, i64, i32, i32, vp], None
        L.csa2o_reindex_topk.argtypes, L.csa2o_reindex_topk.restype = [vp, vp, i32, i64, i64, i32, vp], None
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    assert a.dtype == dtype, (a.dtype, dtype)
    return a


def max_threads() -> int:
    return lib().csa2o_max_threads()


def set_threads(n: int) -> int:
    """Thread count of the oracle's OpenMP loops; returns the previous one."""
    return lib().csa2o_set_threads(int(n))


def e2m1(code: int) -> float:
    return lib().csa2o_e2m1(code)


def e8m0(e: int) -> float:
    return lib().csa2o_e8m0(e)


def dequant_rows(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """codes uint8 [R][dim/2], scales uint8 [R][dim/32] -> float64 [R][dim]."""
    codes, scales = _c(codes, np.uint8), _c(scales, np.uint8)
    R, half = codes.shape
    dim = half * 2
    out = np.empty((R, dim), np.float64)
    L = lib()
    for r in range(R):
        L.csa2o_dequant_row(_ptr(codes[r]), _ptr(scales[r]), dim, _ptr(out[r]))
    return out


def n_visible(pos: int, ratio: int, N: int) -> int:
    return lib().csa2o_n_visible(pos, ratio, N)


def index_score(q: np.ndarray, w: np.ndarray, key: np.ndarray) -> float:
    """q uint16(bf16 bits) [32][128], w float32 [32], key uint16 [128]."""
    q, w, key = _c(q, np.uint16), _c(w, np.float32), _c(key, np.uint16)
    return lib().csa2o_index_score(_ptr(q), _ptr(w), _ptr(key))


def index(q_idx, w_idx, k_idx, q_pos, ratio, q_per_seq):
    """q_idx uint16 [T][32][128], w float32 [T][32], k_idx uint16 [B][N][128],
    q_pos int32 [T] or None -> float64 scores [T][N] (-inf beyond visibility)."""
    q_idx, w_idx, k_idx = _c(q_idx, np.uint16), _c(w_idx, np.float32), _c(k_idx, np.uint16)
    T = q_idx.shape[0]
    N = k_idx.shape[1]
    qp = None if q_pos is None else _c(q_pos, np.int32)
    out = np.empty((T, N), np.float64)
    lib().csa2o_index(_ptr(q_idx), _ptr(w_idx), _ptr(k_idx), _ptr(qp), ratio, T, q_per_seq, N, _ptr(out))
    return out


def index_mx(q_codes, q_scales, w_idx, k_codes, k_scales, q_pos, ratio, q_per_seq):
    """MXFP4 indexer (report sec. 2.4.4): q_codes uint8 [T][32][64], q_scales uint8 [T][32][4],
    w float32 [T][32], k_codes uint8 [B][N][64], k_scales uint8 [B][N][4], q_pos int32 [T] or None
    -> float64 scores [T][N] of the dequantised vectors (-inf beyond visibility)."""
    q_codes, q_scales = _c(q_codes, np.uint8), _c(q_scales, np.uint8)
    k_codes, k_scales, w_idx = _c(k_codes, np.uint8), _c(k_scales, np.uint8), _c(w_idx, np.float32)
    T, N = q_codes.shape[0], k_codes.shape[1]
    qp = None if q_pos is None else _c(q_pos, np.int32)
    out = np.empty((T, N), np.float64)
    lib().csa2o_index_mx(_ptr(q_codes), _ptr(q_scales), _ptr(w_idx), _ptr(k_codes), _ptr(k_scales), _ptr(qp), ratio,
                         T, q_per_seq, N, _ptr(out))
    return out


def topk_row(scores: np.ndarray, n_vis: int, k: int) -> np.ndarray:
    scores = _c(scores, np.float64)
    out = np.empty(k, np.int32)
    lib().csa2o_topk_row(_ptr(scores), n_vis, k, _ptr(out))
    return out


def topk(scores, q_pos, ratio, k):
    scores = _c(scores, np.float64)
    T, N = scores.shape
    qp = None if q_pos is None else _c(q_pos, np.int32)
    out = np.empty((T, k), np.int32)
    lib().csa2o_topk(_ptr(scores), _ptr(qp), ratio, T, N, k, _ptr(out))
    return out


def bf16_round(x: float) -> float:
    """The nearest bf16 value of x (ties to even), as a float."""
    return lib().csa2o_bf16_round(float(x))


def topk_bf16(scores, q_pos, ratio, k):
    """Top-k of the bf16-rounded scores (value desc, index asc), ascending, -1 padded."""
    scores = _c(scores, np.float64)
    T, N = scores.shape
    qp = None if q_pos is None else _c(q_pos, np.int32)
    out = np.empty((T, k), np.int32)
    lib().csa2o_topk_bf16(_ptr(scores), _ptr(qp), ratio, T, N, k, _ptr(out))
    return out


HSI_BLOCK, HSI_BLOCKS = 8, 2048  # report sec. 4.2.1: at most 2048 blocks of 8 positions


def hsi_pool(scores, q_pos, ratio, block=HSI_BLOCK, n_blocks=HSI_BLOCKS):
    """Candidate pool of the hierarchical sparse indexer (report sec. 2.3.2):
    scores float64 [T][N] (a Full layer's) -> int32 [T][n_blocks*block], ascending, -1 padded."""
    scores = _c(scores, np.float64)
    T, N = scores.shape
    qp = None if q_pos is None else _c(q_pos, np.int32)
    out = np.empty((T, n_blocks * block), np.int32)
    lib().csa2o_hsi_pool(_ptr(scores), _ptr(qp), ratio, T, N, block, n_blocks, _ptr(out))
    return out


def reindex_topk(scores, pool, k):
    """Reindex selection (report sec. 2.3.2): top-k of the pool entries by (score desc,
    index asc); scores float64 [T][N] (the Reindex layer's), pool int32 [T][P] -> int32 [T][k]."""
    scores, pool = _c(scores, np.float64), _c(pool, np.int32)
    T, N = scores.shape
    out = np.empty((T, k), np.int32)
    lib().csa2o_reindex_topk(_ptr(scores), _ptr(pool), T, N, pool.shape[1], k, _ptr(out))
    return out


def e4m3(code: int) -> float:
    return lib().csa2o_e4m3(code)


def dequant_rows_e4m3(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """E2M1 codes uint8 [R][D/2] with E4M3 scales uint8 [R][D/16] -> float64 [R][D]."""
    codes, scales = _c(codes, np.uint8), _c(scales, np.uint8)
    R, D = codes.shape[0], codes.shape[1] * 2
    out = np.empty((R, D), np.float64)
    for r in range(R):
        lib().csa2o_dequant_row_e4m3(_ptr(codes[r]), _ptr(scales[r]), D, _ptr(out[r]))
    return out


def dequant_swa_fp8(fp8: np.ndarray, rope: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """FP8 window rows: fp8 uint8 [R][448], rope uint16 [R][64], scales uint8 [R][8] -> float64 [R][512]."""
    fp8, rope, scales = _c(fp8, np.uint8), _c(rope, np.uint16), _c(scales, np.uint8)
    out = np.empty((fp8.shape[0], DIM), np.float64)
    for r in range(fp8.shape[0]):
        lib().csa2o_dequant_swa_fp8_row(_ptr(fp8[r]), _ptr(rope[r]), _ptr(scales[r]), _ptr(out[r]))
    return out


def rope_rotate(v: np.ndarray, pos: float, base: float) -> np.ndarray:
    """Rotate channels 448..511 of a 512-vector by RoPE at position pos (returns a copy)."""
    v = np.array(v, np.float64)
    lib().csa2o_rope_rotate(_ptr(v), float(pos), float(base))
    return v


def attend_ex(q, kv_codes, kv_scales, indices, swa_end, sink, softmax_scale, q_per_seq, window, kv_format=0,
              swa=None, swa_fp8=None, swa_rope=None, swa_scales=None, rope_pos=None, rope_base=10000.0):
    """attend with the main-KV format (0: MXFP4 scales [B][N][16]; 1: E4M3 per 16, scales [B][N][32]),
    the window as bf16 rows (swa uint16 [B][S][512]) or FP8 rows (swa_fp8 uint8 [B][S][448],
    swa_rope uint16 [B][S][64], swa_scales uint8 [B][S][8]), and the optional inverse RoPE of the
    output at -rope_pos[t]."""
    q = _c(q, np.uint16)
    kv_codes, kv_scales = _c(kv_codes, np.uint8), _c(kv_scales, np.uint8)
    indices, swa_end = _c(indices, np.int32), _c(swa_end, np.int32)
    sk = None if sink is None else _c(np.asarray(sink, np.float64), np.float64)
    T, N, k = q.shape[0], kv_codes.shape[1], indices.shape[1]
    if swa is not None:
        swa = _c(swa, np.uint16)
        S, swa_format = swa.shape[1], 0
    else:
        swa_fp8, swa_rope, swa_scales = _c(swa_fp8, np.uint8), _c(swa_rope, np.uint16), _c(swa_scales, np.uint8)
        S, swa_format = swa_fp8.shape[1], 1
    rp = None if rope_pos is None else _c(rope_pos, np.int32)
    out = np.empty((T, HEADS, DIM), np.float64)
    lse = np.empty((T, HEADS), np.float64)
    lib().csa2o_attend_ex(_ptr(q), _ptr(kv_codes), _ptr(kv_scales), kv_format, _ptr(indices), _ptr(swa),
                          _ptr(swa_fp8), _ptr(swa_rope), _ptr(swa_scales), swa_format, _ptr(swa_end), _ptr(sk),
                          float(softmax_scale), T, q_per_seq, N, S, window, k, _ptr(rp), float(rope_base), _ptr(out),
                          _ptr(lse))
    return out, lse


def attend(q, kv_codes, kv_scales, indices, swa, swa_end, sink, softmax_scale, q_per_seq, window):
    """q uint16 [T][64][512]; kv_codes uint8 [B][N][256]; kv_scales uint8 [B][N][16];
    indices int32 [T][k]; swa uint16 [B][S][512]; swa_end int32 [T]; sink float64 [64] or None.
    Returns (out float64 [T][64][512], lse float64 [T][64])."""
    q = _c(q, np.uint16)
    kv_codes, kv_scales = _c(kv_codes, np.uint8), _c(kv_scales, np.uint8)
    indices, swa, swa_end = _c(indices, np.int32), _c(swa, np.uint16), _c(swa_end, np.int32)
    sk = None if sink is None else _c(np.asarray(sink, np.float64), np.float64)
    T = q.shape[0]
    N = kv_codes.shape[1]
    S = swa.shape[1]
    k = indices.shape[1]
    out = np.empty((T, HEADS, DIM), np.float64)
    lse = np.empty((T, HEADS), np.float64)
    lib().csa2o_attend(_ptr(q), _ptr(kv_codes), _ptr(kv_scales), _ptr(indices), _ptr(swa), _ptr(swa_end),
                       _ptr(sk), float(softmax_scale), T, q_per_seq, N, S, window, k, _ptr(out), _ptr(lse))
    return out, lse


def e2m1_encode(v: float) -> int:
    return lib().csa2o_e2m1_encode(float(v))


def e4m3_encode(v: float) -> int:
    return lib().csa2o_e4m3_encode(float(v))


def quantize_mx_row(x: np.ndarray):
    """float64 [512] -> (codes uint8 [256], E8M0 scales uint8 [16]) by the OCP MX rule."""
    x = _c(np.asarray(x, np.float64), np.float64)
    codes, scales = np.zeros(x.size // 2, np.uint8), np.zeros(x.size // 32, np.uint8)
    for b in range(x.size // 32):
        lib().csa2o_quantize_mx_block(_ptr(x[32 * b:]), _ptr(codes[16 * b:]), _ptr(scales[b:]))
    return codes, scales


def quantize_e4m3_row(x: np.ndarray):
    """float64 [512] -> (codes uint8 [256], E4M3 scales uint8 [32])."""
    x = _c(np.asarray(x, np.float64), np.float64)
    codes, scales = np.zeros(x.size // 2, np.uint8), np.zeros(x.size // 16, np.uint8)
    for b in range(x.size // 16):
        lib().csa2o_quantize_e4m3_block(_ptr(x[16 * b:]), _ptr(codes[8 * b:]), _ptr(scales[b:]))
    return codes, scales


def kv_write(h, w_kv, w_z, w_ik, m, pos, rope_base=10000.0, kv_format=0):
    """CSA2 compressor + indexer-K projection + RoPE + cache quantisation (report sec. 2.3, 2.4.4):
    h uint16 [n_ent*m][d], w_kv / w_z uint16 [d][512] (w_z None for m = 1), w_ik uint16 [512][128],
    pos int32 [n_ent] -> dict(entry fp64 [n][512] after RoPE, codes uint8 [n][256], scales uint8
    [n][16 or 32], k fp64 [n][128], k_bf16 uint16 [n][128])."""
    h, w_kv, w_ik = _c(h, np.uint16), _c(w_kv, np.uint16), _c(w_ik, np.uint16)
    wz = None if w_z is None else _c(w_z, np.uint16)
    pos = _c(pos, np.int32)
    d = h.shape[1]
    n = h.shape[0] // m
    entry = np.empty((n, DIM), np.float64)
    codes = np.empty((n, DIM // 2), np.uint8)
    scales = np.empty((n, DIM // (32 if kv_format == 0 else 16)), np.uint8)
    k = np.empty((n, IDX_DIM), np.float64)
    kb = np.empty((n, IDX_DIM), np.uint16)
    lib().csa2o_kv_write(_ptr(h), _ptr(w_kv), _ptr(wz), _ptr(w_ik), d, n, m, _ptr(pos), float(rope_base), kv_format,
                         _ptr(entry), _ptr(codes), _ptr(scales), _ptr(k), _ptr(kb))
    return dict(entry=entry, codes=codes, scales=scales, k=k, k_bf16=kb)
