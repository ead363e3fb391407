"""GPU parity of csa2_kv_write (the CSA2 compressor, indexer-K projection, RoPE and
cache quantisation) against the CPU oracle, through the C ABI.

The device computes in fp32 (bf16 matrix-core products) and the oracle in fp64,
so a quantisation decision may differ only where the oracle's exact value lies
within fp32 rounding of a decision boundary.  The checks below take every code,
scale and bf16 key and require equality, except for decisions whose exact value
is within a relative 1e-4 (elements, scales) or within 1e-2 of a bf16 unit plus
1e-6 (keys: the absolute term covers keys near zero) of the boundary; such
exceptions must also be rare (at most 1 in 1000).  The fp32 error of these sums
is near 1e-7, so the windows are wide of it and still narrow enough that a
wrong rule, index or layout fails everywhere."""
import sys

import numpy as np
import pytest
import torch

import compressed_sparse_attention_02_amd as csa
import csa2_gen as G
import oracle

pytestmark = pytest.mark.gpu
DEV = "cuda"
BF = torch.bfloat16

E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
E2M1_MID = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
REL = 1e-4


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def e4m3_table():
    return np.array([oracle.e4m3(c) for c in range(128)])


E4M3 = None


def unpack(codes):
    """uint8 [n][L/2] -> int [n][L] codes (element 2i in the low nibble of byte i)."""
    c = codes.astype(np.int64)
    out = np.empty((c.shape[0], c.shape[1] * 2), np.int64)
    out[:, 0::2] = c & 15
    out[:, 1::2] = c >> 4
    return out


def e2m1_value(code):
    return np.where(code & 8, -1.0, 1.0) * E2M1[code & 7]


def scale_values(scales, fmt):
    global E4M3
    if fmt == "mx":
        return np.ldexp(1.0, scales.astype(np.int64) - 127)
    if E4M3 is None:
        E4M3 = e4m3_table()
    return E4M3[scales.astype(np.int64) & 127]


def check_quantised(x, codes_g, scales_g, codes_o, scales_o, fmt, what):
    """x fp64 [n][L] (exact pre-quantisation values); *_g device bytes, *_o oracle bytes."""
    blk = 32 if fmt == "mx" else 16
    n, L = x.shape
    xb = x.reshape(n, L // blk, blk)
    amax = np.abs(xb).max(axis=2)
    sg, so = scales_g.astype(np.int64), scales_o.astype(np.int64)
    bad_s = sg != so
    if bad_s.any():
        a = amax[bad_s]
        if fmt == "mx":
            near = np.abs(a / np.exp2(np.round(np.log2(a))) - 1.0) < REL
        else:
            v = a / 6.0
            lo, hi = np.minimum(sg[bad_s], so[bad_s]), np.maximum(sg[bad_s], so[bad_s])
            mid = (scale_values(lo, fmt) + scale_values(hi, fmt)) / 2
            near = (hi - lo == 1) & (np.abs(v - mid) <= REL * v)
        assert near.all(), f"{what}: {int((~near).sum())} scale codes differ away from a boundary"
    cg, co = unpack(codes_g).reshape(n, L // blk, blk), unpack(codes_o).reshape(n, L // blk, blk)
    same_scale = ~bad_s
    diff = (cg != co) & same_scale[:, :, None]
    n_diff = int(diff.sum())
    if n_diff:
        s = scale_values(so, fmt)[:, :, None]
        y = (xb / s)[diff]
        ay = np.abs(y)
        dist = np.abs(ay[:, None] - E2M1_MID[None, :]).min(axis=1)
        zero_sign = (ay < 1e-3) & ((cg[diff] & 7) == 0) & ((co[diff] & 7) == 0)
        ok = (dist <= REL * np.maximum(1.0, ay)) | zero_sign
        assert ok.all(), f"{what}: {int((~ok).sum())} codes differ away from a boundary, e.g. y={y[~ok][:4]}"
    total = int(bad_s.sum()) + n_diff
    assert total <= max(2, x.size // 1000), f"{what}: {total} boundary decisions differ"
    # values: every device element within the format's step of the exact value
    deq = e2m1_value(cg) * scale_values(sg, fmt)[:, :, None]
    assert np.all(np.abs(deq - xb) <= 2.0 * scale_values(sg, fmt)[:, :, None] + 1e-12), what
    return total


def bf16_to_f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def nearest_even_bf16_bits(x):
    """bf16 bit patterns of the fp64 values x rounded once to 8 significant bits, ties to
    the even significand (normal range only, which holds for these keys)."""
    f, e = np.frexp(x)
    r = np.ldexp(np.rint(np.ldexp(f, 8)), e - 8)
    return (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def check_k_bf16(k_gpu_bits, k_exact, k_or_bits, what, atol=1e-6):
    """Device keys (bf16) against the exact keys: within bf16 rounding plus atol (the
    fp32 accumulation error, which dominates for keys near zero), and equal to the
    direct nearest-even rounding of the exact key (which the oracle's bf16 keys are)
    except where the exact key is that close to a rounding midpoint."""
    direct = nearest_even_bf16_bits(k_exact)
    assert np.array_equal(k_or_bits, direct), f"{what}: oracle keys are not the direct rounding"
    kg = bf16_to_f64(k_gpu_bits)
    err = np.abs(kg - k_exact) - 2.0 ** -8 * np.abs(k_exact)
    worst = np.unravel_index(np.argmax(err), err.shape)
    assert err.max() <= atol, f"{what}: at {worst} device {kg[worst]!r} exact {k_exact[worst]!r}"
    diff = k_gpu_bits != direct
    if diff.any():
        k = np.abs(k_exact[diff])
        ulp = np.exp2(np.floor(np.log2(k)) - 7)
        mid = (np.floor(k / ulp) + 0.5) * ulp
        ok = np.abs(k - mid) <= 1e-2 * ulp + atol
        assert ok.all(), f"{what}: keys differ away from a rounding midpoint: {k_exact[diff][~ok][:4]}"
    assert int(diff.sum()) <= max(2, k_exact.size // 1000), what


def run_oracle(inp, m, kv_format, rope_base):
    u = lambda t: None if t is None else t.cpu().numpy().view(np.uint16)
    w_z = None if inp["w_z"] is None else np.ascontiguousarray(u(inp["w_z"]).T)
    return oracle.kv_write(u(inp["h"]), np.ascontiguousarray(u(inp["w_kv"]).T), w_z,
                           np.ascontiguousarray(u(inp["w_ik"]).T), m, inp["pos"].cpu().numpy(), rope_base,
                           kv_format)


def run_gpu(inp, m, kv_format, k_format, rope_base):
    g = {k: (None if v is None else v.to(DEV)) for k, v in inp.items()}
    wz = None if g["w_z"] is None else g["w_z"].view(BF)
    return csa.csa2_kv_write(g["h"].view(BF), g["w_kv"].view(BF), g["w_ik"].view(BF), g["pos"], m=m, w_z=wz,
                             rope_base=rope_base, kv_format=kv_format, k_format=k_format)


def check_case(n_ent, m, d, kv_format, k_format, seed=5, rope_base=10000.0, inp=None):
    log(f"kv_write n_ent={n_ent} m={m} d={d} kv_format={kv_format} k_format={k_format} seed={seed}")
    if inp is None:
        inp = G.kv_write_inputs(seed, n_ent, m, d)
    ref = run_oracle(inp, m, kv_format, rope_base)
    codes, scales, k_out, k_sc = run_gpu(inp, m, kv_format, k_format, rope_base)
    torch.cuda.synchronize()
    fmt = "mx" if kv_format == csa.KV_MXFP4 else "e4m3"
    check_quantised(ref["entry"], codes.cpu().numpy(), scales.cpu().numpy(), ref["codes"], ref["scales"], fmt,
                    "cache")
    if k_format == csa.K_BF16:
        check_k_bf16(k_out.view(torch.int16).cpu().numpy().view(np.uint16), ref["k"], ref["k_bf16"], "indexer K")
    else:
        kc_o = np.empty((n_ent, 64), np.uint8)
        ks_o = np.empty((n_ent, 4), np.uint8)
        for e in range(n_ent):
            kc_o[e], ks_o[e] = oracle.quantize_mx_row(ref["k"][e])
        check_quantised(ref["k"], k_out.cpu().numpy(), k_sc.cpu().numpy(), kc_o, ks_o, "mx", "indexer K (MXFP4)")
    return codes, scales, k_out, k_sc


CASES = [
    # decode: few tokens, hidden dimension split over the GPU
    (4, 1, 5120, csa.KV_MXFP4, csa.K_BF16),
    (64, 1, 5120, csa.KV_E4M3_16, csa.K_MXFP4),
    # pooled entries, ragged last tile (74 tokens)
    (37, 2, 1024, csa.KV_MXFP4, csa.K_MXFP4),
    (9, 4, 512, csa.KV_E4M3_16, csa.K_BF16),
    (5, 8, 256, csa.KV_MXFP4, csa.K_BF16),
    # many tokens: 4 token tiles per projection block, ragged (1030 and 1040 tokens)
    (1030, 1, 512, csa.KV_MXFP4, csa.K_BF16),
    (520, 2, 256, csa.KV_E4M3_16, csa.K_MXFP4),
]


@pytest.mark.parametrize("n_ent,m,d,kvf,kf", CASES)
def test_kv_write_matches_oracle(n_ent, m, d, kvf, kf):
    check_case(n_ent, m, d, kvf, kf)


def test_kv_write_prefill_pooled_full_width():
    """Encoder-style pooling (m = 2) at the model's hidden size with many tokens."""
    check_case(300, 2, 5120, csa.KV_MXFP4, csa.K_BF16, seed=9)


def test_kv_write_deterministic():
    inp = G.kv_write_inputs(3, 64, 2, 1024)
    a = run_gpu(inp, 2, csa.KV_MXFP4, csa.K_MXFP4, 10000.0)
    b = run_gpu(inp, 2, csa.KV_MXFP4, csa.K_MXFP4, 10000.0)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_kv_write_position_zero_and_small_base():
    """pos = 0 leaves the rotated channels as pooled; another base exercises the angle table."""
    inp = G.kv_write_inputs(11, 16, 1, 512)
    inp["pos"] = torch.zeros(16, dtype=torch.int32)
    check_case(16, 1, 512, csa.KV_MXFP4, csa.K_BF16, inp=inp)
    inp = G.kv_write_inputs(12, 16, 2, 512)
    check_case(16, 2, 512, csa.KV_E4M3_16, csa.K_BF16, rope_base=500.0, inp=inp)


def test_kv_write_zero_states():
    """All-zero hidden states: zero entries, MX scale code 127, E4M3 scale 0, zero keys."""
    inp = G.kv_write_inputs(1, 8, 2, 256)
    inp["h"] = torch.zeros_like(inp["h"])
    c, s, k, _ = run_gpu(inp, 2, csa.KV_MXFP4, csa.K_BF16, 10000.0)
    assert int(c.abs().sum()) == 0 and bool((s == 127).all()) and int(k.view(torch.int16).abs().sum()) == 0
    c, s, k, ks = run_gpu(inp, 2, csa.KV_E4M3_16, csa.K_MXFP4, 10000.0)
    assert int(c.sum()) == 0 and int(s.sum()) == 0 and int(k.sum()) == 0 and bool((ks == 127).all())


def test_kv_write_feeds_attention_format():
    """The written MXFP4 cache dequantises to the oracle entries within the format's step
    (the same rows csa2_attend_fp4 reads)."""
    inp = G.kv_write_inputs(21, 32, 1, 1024)
    ref = run_oracle(inp, 1, 0, 10000.0)
    codes, scales, _, _ = run_gpu(inp, 1, csa.KV_MXFP4, csa.K_BF16, 10000.0)
    deq = oracle.dequant_rows(codes.cpu().numpy(), scales.cpu().numpy())
    s = np.repeat(np.ldexp(1.0, scales.cpu().numpy().astype(np.int64) - 127), 32, axis=1)
    assert np.all(np.abs(deq - ref["entry"]) <= 2.0 * s)
