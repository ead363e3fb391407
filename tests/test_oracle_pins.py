"""Pins of the CPU oracle against facts fixed outside it (no GPU).

Each test checks the oracle against something it does not compute itself:
values printed in a format specification or fixed by the pages (golden files),
closed forms, exact rational arithmetic, an independent textbook
implementation, or invariants that any correct implementation satisfies.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import csa2_gen as G

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def _bf16(x):
    """float -> bf16 bits (exact for the values used here)."""
    u = np.array([x], np.float32).view(np.uint32)[0]
    assert u & 0xFFFF == 0, x
    return np.uint16(u >> 16)


def _bf16_val(b):
    return float(np.array([np.uint32(b) << 16], np.uint32).view(np.float32)[0])


# ------------------------------------------------------------------ formats

def test_e2m1_table_matches_spec(oracle_lib):
    for code, val in _golden("e2m1_values.txt"):
        got = oracle_lib.e2m1(int(code))
        assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val)), code


def test_e8m0_scales(oracle_lib):
    for e in range(255):
        assert oracle_lib.e8m0(e) == 2.0 ** (e - 127)
    assert math.isnan(oracle_lib.e8m0(255))


def test_dequant_worked_example(oracle_lib):
    # 64-channel row: byte i packs channel 2i (low nibble) and 2i+1 (high nibble).
    codes = np.zeros((1, 32), np.uint8)
    codes[0, 0] = 0x21     # ch0 = code 1 (0.5), ch1 = code 2 (1.0)
    codes[0, 1] = 0xF7     # ch2 = code 7 (6.0), ch3 = code 15 (-6.0)
    codes[0, 16] = 0x9B    # ch32 = code 11 (-1.5), ch33 = code 9 (-0.5)
    scales = np.array([[127 + 3, 127 - 5]], np.uint8)   # 2^3 for ch 0..31, 2^-5 for ch 32..63
    x = oracle_lib.dequant_rows(codes, scales)[0]
    assert list(x[:4]) == [4.0, 8.0, 48.0, -48.0]
    assert x[32] == -1.5 / 32 and x[33] == -0.5 / 32
    assert np.all(x[4:32] == 0) and np.all(x[34:] == 0)


def _to_bf16_rne(x):
    u = int(np.array([x], np.float32).view(np.uint32)[0])
    return np.uint16((u + 0x7FFF + ((u >> 16) & 1)) >> 16)


def test_quantize_rounding_ties(oracle_lib):
    # generator quantiser (OCP rule) read back through the oracle's dequantiser;
    # a 4.0 element pins the block's shared scale to 2^0, the probe is element 1
    for inp, exp in _golden("e2m1_rounding.txt"):
        blk = np.zeros(512, np.uint16)
        blk[0::32] = _bf16(4.0)
        blk[1] = _to_bf16_rne(float(inp))
        bits = torch.from_numpy(blk.astype(np.int32)).to(torch.int16).view(1, 512)
        codes, scales = G.mxfp4_quantize(bits)
        assert int(scales[0, 0]) == 127
        x = oracle_lib.dequant_rows(codes.numpy(), scales.numpy())[0]
        assert x[1] == float(exp), (inp, x[1])


def test_quantize_dequantize_roundtrip(oracle_lib):
    # values already on the MXFP4 grid come back unchanged; others land on the
    # nearest grid value (error <= half the local grid step, or clipped at 6*scale)
    rng = np.random.default_rng(0)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)
    rows = 64
    mags = grid[rng.integers(1, 8, size=(rows, 512))] * rng.choice([-1, 1], size=(rows, 512))
    mags[:, ::32] = 6.0        # each block's amax = 6 -> scale 2^(2-2) * 2^e
    exps = rng.integers(-8, 8, size=(rows, 16))
    vals = mags * np.repeat(2.0 ** exps, 32, axis=1)
    bits = torch.from_numpy(np.array([[_bf16(v) for v in r] for r in vals], np.uint16).astype(np.int32)).to(torch.int16)
    codes, scales = G.mxfp4_quantize(bits)
    back = oracle_lib.dequant_rows(codes.numpy(), scales.numpy())
    assert np.array_equal(back, vals)
    # generic N(0,1) data: error bound of round-to-nearest on the E2M1 grid
    x = G.normal_bf16(0, 99, 0, rows * 512).view(rows, 512)
    codes, scales = G.mxfp4_quantize(x)
    back = oracle_lib.dequant_rows(codes.numpy(), scales.numpy())
    xf = G.bf16_bits_to_float(x).double().numpy()
    sc = np.repeat(np.array([[2.0 ** (int(e) - 127) for e in r] for r in scales.numpy()]), 32, axis=1)
    r = np.abs(xf) / sc                       # in [0, 8): amax / scale lies in [4, 8)
    step = np.where(r < 2, 0.5, np.where(r < 4, 1.0, 2.0)) * sc
    inside = r <= 6
    assert np.all(np.abs(back - xf)[inside] <= step[inside] / 2)
    assert np.all(back[~inside] == np.sign(xf[~inside]) * 6 * sc[~inside])   # saturation
    assert np.all(np.abs(back) <= 6 * sc)


def test_kv_bytes_closed_form():
    g = dict((k, int(v)) for k, v in _golden("kv_bytes.txt"))
    per_entry = lambda d, grp: d // 2 + d // grp
    assert per_entry(512, 16) == g["main_kv_e4m3_g16"]
    assert per_entry(128, 32) == g["indexer_k_mxfp4"]
    # three encoder Full sources at m = 2 and one decoder Full source at m = 1
    main, idx = per_entry(512, 16), per_entry(128, 32)
    assert Fraction(3 * (main + idx), 2) + (main + idx) == g["global_per_token"]
    main4 = per_entry(512, 32)
    assert main4 == g["main_kv_mxfp4"]
    assert Fraction(3 * (main4 + idx), 2) + (main4 + idx) == g["global_per_token_mxfp4_main"]
    # the layout the hot path reads: 256 code bytes + 16 scale bytes per entry
    c = G.make_case("t", B=1, N=4)
    assert c.kv_codes.shape[-1] + c.kv_scales.shape[-1] == main4


# --------------------------------------------------------------- visibility

def test_visibility_prefill_closed_form(oracle_lib):
    g = dict((k, int(v)) for k, v in _golden("prefill_visibility.txt"))
    nv = [oracle_lib.n_visible(p, 2, 34816) for p in range(65536, 65536 + 4096)]
    assert nv[0] == g["first"] and nv[-1] == g["last"] and sum(nv) == g["sum"]


def test_visibility_small_cases(oracle_lib):
    # ratio 2: tokens {0,1} form entry 0, {2,3} entry 1 ...
    assert [oracle_lib.n_visible(p, 2, 100) for p in range(6)] == [0, 1, 1, 2, 2, 3]
    # ratio 1: the current token's own entry is complete
    assert [oracle_lib.n_visible(p, 1, 100) for p in range(3)] == [1, 2, 3]
    assert oracle_lib.n_visible(10 ** 9, 1, 100) == 100     # capped at N
    assert oracle_lib.n_visible(-1, 4, 77) == 0             # before the first token: nothing


# ------------------------------------------------------------------ indexer

def _exact_score(q_bits, w, key_bits):
    tot = Fraction(0)
    for h in range(32):
        d = sum(Fraction(_bf16_val(q_bits[h, c])) * Fraction(_bf16_val(key_bits[c])) for c in range(128))
        tot += Fraction(float(w[h])) * max(d, Fraction(0))
    return tot


def test_index_score_integer_inputs_exact(oracle_lib):
    # small integers: every fp64 step is exact, so the oracle must equal the
    # integer formula sum_h w_h * max(0, sum_c q[h][c] * k[c]) exactly
    rng = np.random.default_rng(1)
    for trial in range(20):
        qi = rng.integers(-3, 4, size=(32, 128))
        ki = rng.integers(-3, 4, size=128)
        wi = rng.integers(0, 5, size=32)
        q = np.array([[_bf16(float(v)) for v in r] for r in qi], np.uint16)
        k = np.array([_bf16(float(v)) for v in ki], np.uint16)
        w = wi.astype(np.float32)
        exp = sum(int(wi[h]) * max(0, int(np.dot(qi[h], ki))) for h in range(32))
        assert oracle_lib.index_score(q, w, k) == exp


def test_index_score_one_hot_weight(oracle_lib):
    rng = np.random.default_rng(2)
    qi = rng.integers(-3, 4, size=(32, 128))
    ki = rng.integers(-3, 4, size=128)
    q = np.array([[_bf16(float(v)) for v in r] for r in qi], np.uint16)
    k = np.array([_bf16(float(v)) for v in ki], np.uint16)
    for h in range(32):
        w = np.zeros(32, np.float32)
        w[h] = 1.0
        assert oracle_lib.index_score(q, w, k) == max(0, int(np.dot(qi[h], ki)))
    # q = -K on every head: all dot products <= 0 -> score 0
    qn = np.array([[_bf16(-float(v)) for v in ki]] * 32, np.uint16)
    assert oracle_lib.index_score(qn, np.ones(32, np.float32), k) == 0.0


def test_index_score_real_inputs_vs_exact_rational(oracle_lib):
    # N(0,1) bf16 inputs: within fp64 rounding of the exact rational value
    for trial in range(4):
        q = G.normal_bf16(7, 1000 + trial, 0, 32 * 128).view(32, 128).numpy().view(np.uint16)
        k = G.normal_bf16(7, 2000 + trial, 0, 128).numpy().view(np.uint16)
        w = G.uniform_f32(7, 3000 + trial, 0, 32).numpy()
        exact = _exact_score(q, w, k)
        scale = sum(abs(float(w[h])) * sum(abs(_bf16_val(q[h, c]) * _bf16_val(k[c])) for c in range(128))
                    for h in range(32))
        got = oracle_lib.index_score(q, w, k)
        assert abs(Fraction(got) - exact) <= Fraction(scale) * Fraction(1, 2 ** 44)


def test_index_power_of_two_weight_scaling(oracle_lib):
    c = G.make_case("t", B=1, N=300, with_kv=False)
    s1 = oracle_lib.index(c.q_idx.numpy().view(np.uint16), c.w_idx.numpy(), c.k_idx.numpy().view(np.uint16),
                          c.q_pos.numpy(), 1, 1)
    s2 = oracle_lib.index(c.q_idx.numpy().view(np.uint16), c.w_idx.numpy() * 8.0,
                          c.k_idx.numpy().view(np.uint16), c.q_pos.numpy(), 1, 1)
    assert np.array_equal(s1 * 8.0, s2)
    assert np.array_equal(oracle_lib.topk(s1, c.q_pos.numpy(), 1, 64), oracle_lib.topk(s2, c.q_pos.numpy(), 1, 64))


def test_index_batch_layout_and_visibility(oracle_lib):
    # 2 sequences x 3 queries at ratio 2; each query uses its own sequence's keys
    B, qps, N, ratio = 2, 3, 40, 2
    T = B * qps
    q = G.normal_bf16(3, 1, 0, T * 32 * 128).view(T, 32, 128).numpy().view(np.uint16)
    w = G.uniform_f32(3, 2, 0, T * 32).view(T, 32).numpy()
    k = G.normal_bf16(3, 3, 0, B * N * 128).view(B, N, 128).numpy().view(np.uint16)
    pos = np.array([10, 41, 79, 0, 5, 200], np.int32)
    s = oracle_lib.index(q, w, k, pos, ratio, qps)
    for t in range(T):
        nv = min(N, (int(pos[t]) + 1) // ratio)
        for j in range(N):
            if j < nv:
                assert s[t, j] == oracle_lib.index_score(q[t], w[t], k[t // qps, j])
            else:
                assert s[t, j] == -np.inf


# -------------------------------------------------------------------- top-k

def _topk_reference(scores, n_vis, k):
    order = sorted(range(n_vis), key=lambda s: (-scores[s], s))
    sel = sorted(order[:k])
    return sel + [-1] * (k - len(sel))


def test_topk_equals_full_sort(oracle_lib):
    rng = np.random.default_rng(3)
    for n in [1, 7, 511, 512, 513, 2000]:
        sc = rng.normal(size=n)
        assert list(oracle_lib.topk_row(sc, n, 512)) == _topk_reference(list(sc), n, 512)


def test_topk_ties_lower_index_wins(oracle_lib):
    sc = np.zeros(1000)
    sc[::3] = 1.0                  # 334 entries tie at 1.0
    sc[500:] += 0.0                # equal values beyond
    got = list(oracle_lib.topk_row(sc, 1000, 512))
    exp = sorted([i for i in range(0, 1000, 3)] + [i for i in range(1000) if i % 3 != 0][:178])
    assert got == exp
    # all equal: the lowest 512 indices
    assert list(oracle_lib.topk_row(np.full(2048, 3.5), 2048, 512)) == list(range(512))


def test_topk_visibility_and_padding(oracle_lib):
    rng = np.random.default_rng(4)
    sc = rng.normal(size=(3, 700))
    pos = np.array([99, 699, 2000], np.int32)
    out = oracle_lib.topk(sc, pos, 1, 512)
    assert list(out[0]) == list(range(100)) + [-1] * 412
    assert list(out[1]) == _topk_reference(list(sc[1]), 700, 512)
    assert list(out[2]) == _topk_reference(list(sc[2]), 700, 512)


# ---------------------------------------------------------------- attention

def _dense_attention(q, rows, scale, sink=None):
    """Textbook softmax attention with key = value = rows (numpy, fp64)."""
    z = scale * (q @ rows.T)                       # [H][n]
    if sink is not None:
        z = np.concatenate([z, np.asarray(sink)[:, None]], axis=1)
        vals = np.concatenate([rows, np.zeros((1, rows.shape[1]))], axis=0)
    else:
        vals = rows
    m = z.max(axis=1, keepdims=True)
    p = np.exp(z - m)
    out = (p / p.sum(axis=1, keepdims=True)) @ vals
    lse = (m[:, 0] + np.log(p.sum(axis=1)))
    return out, lse


def _bits_to_f64(b):
    return G.bf16_bits_to_float(torch.from_numpy(np.ascontiguousarray(b).view(np.int16))).double().numpy()


def test_attend_dense_case_matches_textbook(oracle_lib):
    # every entry selected (k >= N): sparse attention reduces to dense attention
    c = G.make_case("t", B=2, N=40, q_per_seq=2, window=16, seed=5)
    T = c.T
    idx = np.tile(np.arange(40, dtype=np.int32), (T, 1))
    idx = np.concatenate([idx, -np.ones((T, 8), np.int32)], axis=1)    # some empty slots
    q = c.q[0].numpy().view(np.uint16)
    swa = c.swa[0].numpy().view(np.uint16)
    swa_end = np.array([16, 9, 16, 1], np.int32)
    sink = np.linspace(-1, 2, 64)
    for sk in (None, sink):
        out, lse = oracle_lib.attend(q, c.kv_codes.numpy(), c.kv_scales.numpy(), idx, swa, swa_end, sk,
                                     0.07, 2, 16)
        for t in range(T):
            b = t // 2
            kv = oracle_lib.dequant_rows(c.kv_codes[b].numpy(), c.kv_scales[b].numpy())
            e = int(swa_end[t])
            win = _bits_to_f64(swa[b, max(0, e - 16):e])
            rows = np.concatenate([kv, win], axis=0)
            ref, rlse = _dense_attention(_bits_to_f64(q[t]), rows, 0.07, sk)
            np.testing.assert_allclose(out[t], ref, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(lse[t], rlse, rtol=1e-12, atol=1e-12)


def test_attend_degenerate_cases(oracle_lib):
    c = G.make_case("t", B=1, N=16, window=4, seed=6)
    q = c.q[0].numpy().view(np.uint16)
    swa = c.swa[0].numpy().view(np.uint16)
    kv = oracle_lib.dequant_rows(c.kv_codes[0].numpy(), c.kv_scales[0].numpy())
    # one selected entry, no window: output = that entry, lse = its logit
    idx = np.array([[-1, 5, -1, -1]], np.int32)
    out, lse = oracle_lib.attend(q, c.kv_codes.numpy(), c.kv_scales.numpy(), idx, swa, np.array([0], np.int32),
                                 None, 0.1, 1, 4)
    assert np.allclose(out[0], np.broadcast_to(kv[5], (64, 512)), rtol=0, atol=0)
    np.testing.assert_allclose(lse[0], 0.1 * (_bits_to_f64(q[0]) @ kv[5]), rtol=1e-13)
    # the same entry selected several times: still that entry
    idx = np.array([[5, 5, 5, 5]], np.int32)
    out, _ = oracle_lib.attend(q, c.kv_codes.numpy(), c.kv_scales.numpy(), idx, swa, np.array([0], np.int32),
                               None, 0.1, 1, 4)
    np.testing.assert_allclose(out[0], np.broadcast_to(kv[5], (64, 512)), rtol=1e-14)
    # a sink of -inf is the same as no sink
    idx = np.array([[0, 3, 9, 15]], np.int32)
    a, la = oracle_lib.attend(q, c.kv_codes.numpy(), c.kv_scales.numpy(), idx, swa, np.array([4], np.int32),
                              None, 0.1, 1, 4)
    b, lb = oracle_lib.attend(q, c.kv_codes.numpy(), c.kv_scales.numpy(), idx, swa, np.array([4], np.int32),
                              np.full(64, -np.inf), 0.1, 1, 4)
    assert np.array_equal(a, b) and np.array_equal(la, lb)
    # output lies in the convex hull of the attended rows (per channel)
    rows = np.concatenate([kv[[0, 3, 9, 15]], _bits_to_f64(swa[0, 0:4])], axis=0)
    assert np.all(a >= rows.min(axis=0) - 1e-12) and np.all(a <= rows.max(axis=0) + 1e-12)


def test_attend_window_bounds(oracle_lib):
    # rows outside [end - W, end) must not matter: plant huge values there
    c = G.make_case("t", B=1, N=8, window=4, seed=8)
    c.S = 12
    swa = G.normal_bf16(8, 77, 0, 12 * 512).view(1, 12, 512).numpy().view(np.uint16).copy()
    q = c.q[0].numpy().view(np.uint16)
    idx = np.array([[1, 2]], np.int32)
    end = np.array([9], np.int32)
    base, _ = oracle_lib.attend(q, c.kv_codes.numpy(), c.kv_scales.numpy(), idx, swa, end, None, 0.05, 1, 4)
    planted = swa.copy()
    planted[0, :5] = _bf16(100.0)
    planted[0, 9:] = _bf16(-100.0)
    got, _ = oracle_lib.attend(q, c.kv_codes.numpy(), c.kv_scales.numpy(), idx, planted, end, None, 0.05, 1, 4)
    assert np.array_equal(base, got)
    # and a row inside the window does matter
    planted = swa.copy()
    planted[0, 5] = _bf16(3.0)
    got, _ = oracle_lib.attend(q, c.kv_codes.numpy(), c.kv_scales.numpy(), idx, planted, end, None, 0.05, 1, 4)
    assert not np.array_equal(base, got)


def test_reuse_is_attention_with_new_query(oracle_lib):
    # Reuse (V4.1 report sec. 2.3.1) attends the Full layer's selection with
    # its own query and window; with the Full layer's query it reproduces the
    # Full layer's output, with another query the output changes.
    c = G.make_case("t", B=1, N=64, window=8, n_layers=2, seed=9)
    idx = np.arange(0, 64, 2, dtype=np.int32)[None, :]
    args = (c.kv_codes.numpy(), c.kv_scales.numpy(), idx)
    full, _ = oracle_lib.attend(c.q[0].numpy().view(np.uint16), *args, c.swa[0].numpy().view(np.uint16),
                                c.swa_end.numpy(), None, 0.04, 1, 8)
    again, _ = oracle_lib.attend(c.q[0].numpy().view(np.uint16), *args, c.swa[0].numpy().view(np.uint16),
                                 c.swa_end.numpy(), None, 0.04, 1, 8)
    other, _ = oracle_lib.attend(c.q[1].numpy().view(np.uint16), *args, c.swa[1].numpy().view(np.uint16),
                                 c.swa_end.numpy(), None, 0.04, 1, 8)
    assert np.array_equal(full, again) and not np.allclose(full, other)


# ---- hierarchical sparse indexer (candidate pool) and Reindex, report sec. 2.3.2

def test_hsi_pool_hand_example(oracle_lib):
    import oracle
    row = np.zeros(27, np.float64)
    row[[3, 9, 14, 20, 24, 26]] = [5, 7, 7, 5, -1, 6]
    for r in _golden("hsi_pool_example.txt"):
        n_vis, n_blocks = int(r[0]), int(r[1])
        want = [int(x) for x in r[3:]]
        out = np.empty(n_blocks * 8, np.int32)
        cnt = oracle.lib().csa2o_hsi_pool_row(oracle._ptr(row), n_vis, 8, n_blocks, oracle._ptr(out))
        assert cnt == len(want) and list(out[:cnt]) == want and np.all(out[cnt:] == -1), (n_vis, n_blocks)


def _pool_brute(row, n_vis, block, n_blocks):
    """Independent loops: block scores, then blocks ranked by (score desc, block asc)."""
    nb = -(-n_vis // block)
    best = []
    for b in range(nb):
        m = max(row[e] for e in range(b * block, min(b * block + block, n_vis)))
        best.append((-m, b))
    chosen = sorted(b for _, b in sorted(best)[:n_blocks])
    return [e for b in chosen for e in range(b * block, min(b * block + block, n_vis))]


def test_hsi_pool_brute_force_small(oracle_lib):
    import oracle
    rng = np.random.default_rng(5)
    for trial in range(40):
        N = int(rng.integers(1, 200))
        n_blocks = int(rng.integers(1, 12))
        # coarse values so that block scores tie often
        s = rng.integers(-3, 4, size=(3, N)).astype(np.float64)
        q_pos = np.array([N - 1, int(rng.integers(-1, N)), int(rng.integers(0, 2 * N))], np.int32)
        pool = oracle.hsi_pool(s, q_pos, 1, 8, n_blocks)
        for t in range(3):
            nv = max(0, min(N, int(q_pos[t]) + 1))
            want = _pool_brute(s[t], nv, 8, n_blocks) if nv else []
            got = pool[t][pool[t] >= 0]
            assert list(got) == want and np.all(pool[t][len(want):] == -1), (trial, t)


def test_hsi_pool_small_rows_are_everything(oracle_lib):
    import oracle
    rng = np.random.default_rng(6)
    s = rng.standard_normal((2, 16384))
    pool = oracle.hsi_pool(s, np.array([16383, 9000], np.int32), 1)
    assert np.array_equal(pool[0], np.arange(16384))
    assert np.array_equal(pool[1][:9001], np.arange(9001)) and np.all(pool[1][9001:] == -1)


def test_hsi_pool_planted_blocks(oracle_lib):
    import oracle
    rng = np.random.default_rng(7)
    N = 50000
    s = rng.standard_normal((1, N))
    planted = [17, 900, 3000, 6249]
    for b in planted:
        s[0, 8 * b + int(rng.integers(0, 8))] = 100.0 + b
    pool = oracle.hsi_pool(s, None, 1, 8, len(planted))
    want = [e for b in sorted(planted) for e in range(8 * b, 8 * b + 8)]
    assert list(pool[0][pool[0] >= 0]) == want


def test_reindex_with_full_query_reproduces_full_topk(oracle_lib):
    """The pool contains every block holding a Full top-k entry (at most k <= 2048 blocks,
    and each of them outranks every block without one), so a Reindex layer that scored
    with the Full layer's own query would select exactly the Full top-k."""
    import oracle
    rng = np.random.default_rng(8)
    for N, ties in [(40000, False), (30000, True), (20000, True)]:
        s = rng.standard_normal((3, N))
        if ties:
            s = np.round(s, 1)  # many equal scores, also across block boundaries
        q_pos = np.array([N - 1, N // 2, 16000], np.int32)
        full = oracle.topk(s, q_pos, 1, 512)
        pool = oracle.hsi_pool(s, q_pos, 1)
        for t in range(3):
            assert set(full[t][full[t] >= 0]) <= set(pool[t][pool[t] >= 0])
        assert np.array_equal(oracle.reindex_topk(s, pool, 512), full)


def test_reindex_topk_brute_force(oracle_lib):
    import oracle
    rng = np.random.default_rng(9)
    N, k = 3000, 64
    s_full = rng.standard_normal((2, N))
    s_re = np.round(rng.standard_normal((2, N)), 1)
    pool = oracle.hsi_pool(s_full, None, 1, 8, 40)
    got = oracle.reindex_topk(s_re, pool, k)
    for t in range(2):
        cand = [int(e) for e in pool[t] if e >= 0]
        want = sorted(sorted(cand, key=lambda e: (-s_re[t, e], e))[:k])
        assert list(got[t][:len(want)]) == want and np.all(got[t][len(want):] == -1)
        assert set(want) <= set(cand)


# ---- MXFP4 indexer queries and keys (report sec. 2.4.4: FP4 indexer q/K, MXFP4)

def _mx_vec(values_by_channel, scales):
    """Hand-built 128-channel MXFP4 vector: {channel: E2M1 code}, 4 scale bytes."""
    codes = np.zeros(64, np.uint8)
    for c, code in values_by_channel.items():
        codes[c // 2] |= np.uint8(code << (4 * (c % 2)))
    return codes, np.array(scales, np.uint8)


def test_index_mx_hand_worked_channel_placement(oracle_lib):
    # q head 0: channel 33 = E2M1 code 7 (6.0) in scale block 1 (2^(128-127) = 2) -> 12.0
    # key:      channel 33 = code 3 (1.5), block 1 scale 2^(126-127) -> 0.75; dot = 9.0
    # a key holding the same value at channel 32 instead contributes nothing
    import oracle
    qc = np.zeros((1, 32, 64), np.uint8)
    qs = np.full((1, 32, 4), 127, np.uint8)
    c0, s0 = _mx_vec({33: 7}, [127, 128, 127, 127])
    qc[0, 0], qs[0, 0] = c0, s0
    w = np.zeros((1, 32), np.float32)
    w[0, 0] = 1.0
    kc = np.zeros((1, 2, 64), np.uint8)
    ks = np.full((1, 2, 4), 127, np.uint8)
    kc[0, 0], ks[0, 0] = _mx_vec({33: 3}, [127, 126, 127, 127])
    kc[0, 1], ks[0, 1] = _mx_vec({32: 3}, [127, 126, 127, 127])
    s = oracle.index_mx(qc, qs, w, kc, ks, None, 1, 1)
    assert s[0, 0] == 9.0 and s[0, 1] == 0.0


def test_index_mx_closed_form(oracle_lib):
    # every channel of head h is 1.0 (code 2) times 2^a_h with sign (-1)^h, every channel
    # of key s is 0.5 (code 1) times 2^b_s: dot = +-128 * 0.5 * 2^(a_h + b_s);
    # score = sum over even heads of w_h * 64 * 2^(a_h + b_s) (odd heads are negative -> 0)
    import oracle
    rng = np.random.default_rng(3)
    a = rng.integers(-6, 7, 32)
    b = rng.integers(-6, 7, 5)
    qc = np.zeros((1, 32, 64), np.uint8)
    qs = np.zeros((1, 32, 4), np.uint8)
    for h in range(32):
        code = 2 | (8 if h % 2 else 0)
        qc[0, h] = code | (code << 4)
        qs[0, h] = 127 + a[h]
    kc = np.full((1, 5, 64), 1 | (1 << 4), np.uint8)
    ks = np.zeros((1, 5, 4), np.uint8)
    for s in range(5):
        ks[0, s] = 127 + b[s]
    w = (rng.integers(1, 9, (1, 32)) / 8.0).astype(np.float32)
    got = oracle.index_mx(qc, qs, w, kc, ks, None, 1, 1)[0]
    for s in range(5):
        exact = sum(Fraction(float(w[0, h])) * 64 * Fraction(2) ** int(a[h] + b[s]) for h in range(0, 32, 2))
        assert got[s] == float(exact)


def test_index_mx_is_bf16_index_of_dequantised_values(oracle_lib):
    # the FP4 path is the bf16 path on the dequantised vectors (every E2M1 value times a
    # moderate power of two is exact in bf16): the generator's quantised N(0,1) data
    import oracle
    x = G.normal_bf16(7, 1, 0, 3 * 32 * 128).view(3 * 32, 128)
    k = G.normal_bf16(7, 3, 0, 40 * 128).view(40, 128)
    qc, qs = G.mxfp4_quantize(x)
    kc, ks = G.mxfp4_quantize(k)
    deq_q = oracle.dequant_rows(qc.numpy(), qs.numpy())
    deq_k = oracle.dequant_rows(kc.numpy(), ks.numpy())
    to_bf16 = lambda d: np.array([_bf16(v) for v in d.reshape(-1)], np.uint16).reshape(d.shape)
    w = G.uniform_f32(7, 2, 0, 3 * 32).view(3, 32).numpy()
    pos = np.array([39, 20, 7], np.int32)
    ref = oracle.index(to_bf16(deq_q).reshape(3, 32, 128), w, to_bf16(deq_k).reshape(1, 40, 128), pos, 1, 3)
    got = oracle.index_mx(qc.numpy().reshape(3, 32, 64), qs.numpy().reshape(3, 32, 4), w,
                          kc.numpy().reshape(1, 40, 64), ks.numpy().reshape(1, 40, 4), pos, 1, 3)
    assert np.array_equal(got, ref)


# ---- the pages' main-KV format, FP8 window rows, inverse RoPE of the output

def test_e4m3_table_matches_spec(oracle_lib):
    import oracle
    for code, val in _golden("e4m3_values.txt"):
        got = oracle.e4m3(int(code, 16))
        if val == "nan":
            assert math.isnan(got)
        else:
            assert got == float(val) and math.copysign(1.0, got) == math.copysign(1.0, float(val)), (code, got)
    # every finite positive code is larger than the one before; negatives mirror them
    pos = [oracle.e4m3(c) for c in range(0x7F)]
    assert all(b > a for a, b in zip(pos, pos[1:]))
    assert all(oracle.e4m3(0x80 | c) == -oracle.e4m3(c) for c in range(1, 0x7F))


def test_dequant_e4m3_worked_example(oracle_lib):
    # channel 0: code 15 (-6) with scale 0x7E (448) -> -2688, the largest magnitude of the
    # format (report sec. 2.4.4); channel 17 (block 1, high nibble of byte 8): code 5 (3.0)
    # with scale 0x39 (1.125) -> 3.375
    import oracle
    codes = np.zeros((1, 256), np.uint8)
    scales = np.full((1, 32), 0x38, np.uint8)
    codes[0, 0] = 15
    scales[0, 0] = 0x7E
    codes[0, 8] = 5 << 4
    scales[0, 1] = 0x39
    x = oracle.dequant_rows_e4m3(codes, scales)[0]
    want = np.zeros(512)
    want[0], want[17] = -2688.0, 3.375
    assert np.array_equal(x, want)


def test_dequant_swa_fp8_worked_example(oracle_lib):
    # channel 70 (scale block 1): 0x40 (2.0) x 2^(126-127) = 1.0; channel 447 (block 6):
    # 0xB8 (-1.0) x 2^3 = -8; channel 448: bf16 1.5 (the RoPE channels are bf16)
    import oracle
    fp8 = np.zeros((1, 448), np.uint8)
    rope = np.zeros((1, 64), np.uint16)
    sc = np.full((1, 8), 127, np.uint8)
    fp8[0, 70], sc[0, 1] = 0x40, 126
    fp8[0, 447], sc[0, 6] = 0xB8, 130
    rope[0, 0] = _bf16(1.5)
    x = oracle.dequant_swa_fp8(fp8, rope, sc)[0]
    want = np.zeros(512)
    want[70], want[447], want[448] = 1.0, -8.0, 1.5
    assert np.array_equal(x, want)


def _rope_np(v, pos, base):
    """Forward RoPE on channels 448..511 (independent numpy statement of the reading)."""
    v = np.array(v, np.float64)
    j = np.arange(32)
    phi = pos * base ** (-2.0 * j / 64.0)
    x, y = v[..., 448::2].copy(), v[..., 449::2].copy()
    v[..., 448::2] = x * np.cos(phi) - y * np.sin(phi)
    v[..., 449::2] = x * np.sin(phi) + y * np.cos(phi)
    return v


def test_rope_rotate_cases(oracle_lib):
    import oracle
    rng = np.random.default_rng(5)
    v = rng.standard_normal(512)
    assert np.array_equal(oracle.rope_rotate(v, 0.0, 10000.0), v)           # position 0: identity
    e = np.zeros(512)
    e[448] = 1.0                                                             # pair 0, theta = 1
    r = oracle.rope_rotate(e, 1.0, 10000.0)
    assert r[448] == math.cos(1.0) and r[449] == math.sin(1.0)
    e = np.zeros(512)
    e[449 + 32] = 1.0                                                        # pair 16: theta = 10000^-0.5
    r = oracle.rope_rotate(e, 3.0, 10000.0)
    assert abs(r[448 + 32] + math.sin(0.03)) < 1e-15 and abs(r[449 + 32] - math.cos(0.03)) < 1e-15
    r = oracle.rope_rotate(v, 12345.0, 10000.0)
    assert np.array_equal(r[:448], v[:448])                                  # only the last 64 channels
    n = lambda a: np.hypot(a[448::2], a[449::2])
    assert np.allclose(n(r), n(v), rtol=1e-14)                               # pairs keep their norms
    assert np.allclose(oracle.rope_rotate(r, -12345.0, 10000.0), v, atol=1e-12)
    assert np.allclose(r, _rope_np(v, 12345.0, 10000.0), atol=1e-12)


def test_attend_inverse_rope_gives_relative_positions(oracle_lib):
    # every attention row is a value rotated at its own position p_j and the query is rotated
    # at i: scores depend on i - p_j only, and the output rotated at -i is a sum of values
    # rotated by p_j - i.  Shifting every position by the same amount changes nothing.
    import oracle
    rng = np.random.default_rng(9)
    n, W = 6, 4
    base_rows = rng.standard_normal((n + W, 512)) * 0.5
    q_base = rng.standard_normal((64, 512)) * 0.3
    pos_main = rng.integers(0, 50, n)
    pos_win = np.arange(60, 60 + W)
    outs = []
    for shift in (0, 1000):
        i = 70 + shift
        rows = np.stack([_rope_np(base_rows[j], (pos_main[j] if j < n else pos_win[j - n]) + shift, 10000.0)
                         for j in range(n + W)])
        # every row goes through the bf16 window path (n + W window rows, no selected rows):
        # FP4 codes could not hold rotated values
        q = _rope_np(q_base, i, 10000.0)
        to_b = lambda a: (np.asarray(a, np.float32).view(np.uint32) + 0x8000 >> 16).astype(np.uint16)
        swa = to_b(rows)[None]
        qb = to_b(q)[None]
        idx = np.full((1, 512), -1, np.int32)
        kvc = np.zeros((1, 1, 256), np.uint8)
        kvs = np.full((1, 1, 16), 127, np.uint8)
        out, _ = oracle.attend_ex(qb, kvc, kvs, idx, np.array([n + W], np.int32), None, 0.05, 1, n + W, swa=swa,
                                  rope_pos=np.array([i], np.int32), rope_base=10000.0)
        outs.append(out)
    # bf16 rounding of the rotated inputs differs between the two shifts: compare loosely
    assert np.allclose(outs[0], outs[1], atol=2e-2, rtol=2e-2)
    # and without the inverse rotation the last 64 channels do depend on the shift
    assert not np.allclose(_rope_np(outs[0], 70, 10000.0)[..., 448:], _rope_np(outs[1], 1070, 10000.0)[..., 448:],
                           atol=2e-2)


def test_attend_ex_formats_reduce_to_known_cases(oracle_lib):
    # E4M3 scales of exactly 1.0 give the MXFP4 rows with scale 2^0; FP8 window rows whose values
    # are exact with scale 2^0 give the bf16 window path
    import oracle
    rng = np.random.default_rng(11)
    T, B, N, S = 2, 1, 40, 8
    q = (rng.uniform(-1, 1, (T, 64, 512)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    codes = rng.integers(0, 256, (B, N, 256)).astype(np.uint8)
    idx = np.stack([rng.permutation(N)[:12] for _ in range(T)]).astype(np.int32)
    idx = np.concatenate([idx, np.full((T, 500), -1, np.int32)], axis=1)
    swa_end = np.array([8, 5], np.int32)
    fp8 = rng.integers(0, 0x7F, (B, S, 448)).astype(np.uint8)             # finite E4M3 codes
    rope = (rng.uniform(-2, 2, (B, S, 64)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    swa_vals = np.concatenate([np.vectorize(oracle.e4m3)(fp8), np.zeros((B, S, 64))], axis=2)
    swa_bf = (swa_vals.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    swa_bf[..., 448:] = rope
    a, la = oracle.attend_ex(q, codes, np.full((B, N, 16), 127, np.uint8), idx, swa_end, None, 0.04, 2, 8,
                             kv_format=0, swa=swa_bf)
    b, lb = oracle.attend_ex(q, codes, np.full((B, N, 32), 0x38, np.uint8), idx, swa_end, None, 0.04, 2, 8,
                             kv_format=1, swa_fp8=fp8, swa_rope=rope, swa_scales=np.full((B, S, 8), 127, np.uint8))
    assert np.array_equal(a, b) and np.array_equal(la, lb)


# ---- KV write path: compressor, indexer-K projection, RoPE, cache quantisation

def test_e2m1_encode_matches_ocp_ties(oracle_lib):
    import oracle
    grid = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    for inp, exp in _golden("e2m1_rounding.txt"):
        code = oracle.e2m1_encode(float(inp))
        val = grid[code & 7] * (-1 if code & 8 else 1)
        assert val == float(exp), (inp, val)


def test_e4m3_encode_roundtrip_and_ties(oracle_lib):
    import oracle
    for c in range(0x7F):
        v = oracle.e4m3(c)
        assert oracle.e4m3_encode(v) == c
        if c:
            assert oracle.e4m3_encode(-v) == c | 0x80
    for c in range(0x7E):
        mid = (oracle.e4m3(c) + oracle.e4m3(c + 1)) / 2
        assert oracle.e4m3_encode(mid) == (c if c % 2 == 0 else c + 1)
    assert oracle.e4m3_encode(1e9) == 0x7E and oracle.e4m3_encode(-1e9) == 0xFE


def test_quantizers_agree_with_generator_rules(oracle_lib):
    # two independent statements of the same published rules: the generator's (torch) and
    # the oracle's (C) quantisers give identical bytes on N(0,1) bf16 data
    import oracle
    x = G.normal_bf16(13, 5, 0, 16 * 512).view(16, 512)
    xf = G.bf16_bits_to_float(x).double().numpy()
    gc, gs = G.mxfp4_quantize(x)
    ec, es = G.e4m3_16_quantize(x)
    for r in range(16):
        c, s = oracle.quantize_mx_row(xf[r])
        assert np.array_equal(c, gc[r].numpy()) and np.array_equal(s, gs[r].numpy())
        c, s = oracle.quantize_e4m3_row(xf[r])
        assert np.array_equal(c, ec[r].numpy()) and np.array_equal(s, es[r].numpy())
    # a block whose largest magnitude is 6 * 2^k gets scale code 127 + k and is represented exactly
    v = np.zeros(512)
    v[:32] = 6.0 * 2.0 ** -3
    v[1] = -1.5 * 2.0 ** -3
    c, s = oracle.quantize_mx_row(v)
    assert s[0] == 124 and np.array_equal(oracle.dequant_rows(c[None], s[None])[0][:32], v[:32])


def _bits(a):
    return (np.asarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_kv_write_closed_forms(oracle_lib):
    import oracle
    rng = np.random.default_rng(21)
    d, n = 512, 6
    eye = _bits(np.eye(d, 512))
    w_ik = np.zeros((512, 128), np.float32)
    w_ik[:128, :] = np.eye(128)
    w_ik = _bits(w_ik)
    h1 = _bits(rng.uniform(-2, 2, (n, d)))
    hval = (h1.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    pos0 = np.zeros(n, np.int32)
    # m = 1, W_kv = I, position 0: the entry is the token's vector; K its first 128 channels
    r = oracle.kv_write(h1, eye, None, w_ik, 1, pos0)
    assert np.array_equal(r["entry"], hval) and np.array_equal(r["k"], hval[:, :128])
    assert np.array_equal(r["k_bf16"], h1[:, :128])
    # the cache holds the OCP MX quantisation of the entry
    for e in range(n):
        c, s = oracle.quantize_mx_row(r["entry"][e])
        assert np.array_equal(c, r["codes"][e]) and np.array_equal(s, r["scales"][e])
    # RoPE at the entry's position on the last 64 channels only, after K is taken
    pos = rng.integers(0, 100000, n).astype(np.int32)
    rp = oracle.kv_write(h1, eye, None, w_ik, 1, pos, 10000.0, 1)
    for e in range(n):
        assert np.array_equal(rp["entry"][e], oracle.rope_rotate(hval[e], float(pos[e]), 10000.0))
        c, s = oracle.quantize_e4m3_row(rp["entry"][e])
        assert np.array_equal(c, rp["codes"][e]) and np.array_equal(s, rp["scales"][e])
    assert np.array_equal(rp["k"], hval[:, :128])
    # m = 2 with zero gate weights: equal weights, the entry is the mean of the two tokens
    h2 = _bits(rng.uniform(-2, 2, (2 * n, d)))
    h2v = (h2.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    zero = np.zeros((d, 512), np.uint16)
    r2 = oracle.kv_write(h2, eye, zero, w_ik, 2, pos0)
    assert np.allclose(r2["entry"], (h2v[0::2] + h2v[1::2]) / 2, rtol=1e-15, atol=0)
    # a gate that strongly prefers the first token of each pair: the entry is that token
    gate = np.zeros((d, 512), np.float32)
    gate[0, :] = 1.0
    h3 = h2v.copy()
    h3[0::2, 0], h3[1::2, 0] = 60.0, -60.0
    h3b = _bits(h3)
    h3v = (h3b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    r3 = oracle.kv_write(h3b, eye, _bits(gate), w_ik, 2, pos0)
    assert np.allclose(r3["entry"], h3v[0::2], rtol=1e-12, atol=1e-12)


def test_kv_write_key_rounds_once_from_the_exact_sum(oracle_lib):
    """The bf16 indexer key is the nearest-even rounding of the exact (fp64) projection,
    taken once.  Keys built from three exact terms (identity W_kv, unit W_ik weights on
    channels 0..2) land on either side of bf16 midpoints by 2^-30, an offset that fp32
    cannot hold: rounding through fp32 first would turn them into ties and pick the even
    neighbour instead.  Expected bit patterns worked by hand (bf16 of 1 is 0x3F80, one
    bf16 step at 1 is 2^-7)."""
    import oracle
    d = 512
    eye = _bits(np.eye(d, 512))
    cases = [  # (channel 0, 1, 2 of the entry) -> key bits
        ((1.0, 2.0 ** -8, 2.0 ** -30), 0x3F81),      # just above the midpoint 1 + 2^-8: up
        ((1.0, 2.0 ** -8, -2.0 ** -30), 0x3F80),     # just below it: down
        ((1.0, 2.0 ** -8, 0.0), 0x3F80),             # the midpoint itself: to the even 1.0
        ((1.0, 3 * 2.0 ** -8, 0.0), 0x3F82),         # midpoint 1 + 3*2^-8: to the even 1 + 2^-6
        ((1.0, 3 * 2.0 ** -8, -2.0 ** -30), 0x3F81), # just below that midpoint: down to 1 + 2^-7
        ((-1.0, -2.0 ** -8, -2.0 ** -30), 0xBF81),   # the sign is symmetric
        ((2.0 ** 20, 2.0 ** 12, 2.0 ** -8), 0x4981),  # 2^20 + 2^12 + 2^-8: above the tie, up to 2^20 + 2^13
    ]
    n = len(cases)
    h = np.zeros((n, d), np.float32)
    for e, (vals, _) in enumerate(cases):
        h[e, :3] = vals
    hb = _bits(h)
    assert np.array_equal((hb.astype(np.uint32) << 16).view(np.float32), h)   # the terms are bf16 values
    w_ik = np.zeros((512, 128), np.float32)
    w_ik[:3, 0] = 1.0
    r = oracle.kv_write(hb, eye, None, _bits(w_ik), 1, np.zeros(n, np.int32))
    for e, (vals, want) in enumerate(cases):
        assert r["k"][e, 0] == sum(vals)
        assert int(r["k_bf16"][e, 0]) == want, (vals, hex(int(r["k_bf16"][e, 0])), hex(want))
    assert not r["k_bf16"][:, 1:].any()


def test_bf16_round_golden(oracle_lib):
    """The score rounding of the BF16 selector: hand-worked values, ties, the binade carry,
    the sub-normal quantum, overflow, and one case that fp32-then-bf16 would round differently."""
    import oracle
    for inp, exp, *_ in _golden("bf16_rounding.txt"):
        x = float.fromhex(inp)
        want = float("inf") if exp == "inf" else float.fromhex(exp)
        assert oracle.bf16_round(x) == want, (inp, oracle.bf16_round(x), exp)
        assert oracle.bf16_round(-x) == -want


def test_bf16_round_matches_torch_on_fp32_values(oracle_lib):
    """On fp32 inputs direct rounding equals torch's float32 -> bfloat16 conversion (nearest even),
    including planted exact ties (low 16 bits 0x8000) and their neighbours."""
    import oracle
    import torch
    rng = np.random.default_rng(33)
    u = rng.integers(0x00800000, 0x7F000000, 4000, dtype=np.uint32)
    u[:1000] = (u[:1000] & 0xFFFF0000) | 0x8000
    u[1000:1500] = (u[1000:1500] & 0xFFFF0000) | 0x7FFF
    u[1500:2000] = (u[1500:2000] & 0xFFFF0000) | 0x8001
    sign = rng.integers(0, 2, u.size).astype(np.uint32) << 31
    x = (u | sign).view(np.float32)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.bf16_round(float(v)) for v in x])
    assert np.array_equal(got, ref)


def test_topk_bf16_ties_go_to_lower_index(oracle_lib):
    """Scores that differ only below bf16 resolution tie after rounding, and the lower index
    wins; scores a bf16 step apart keep their order."""
    import oracle
    N, k = 40, 6
    s = np.full(N, 0.25)                        # clearly out
    s[[3, 30]] = [8.0, 4.0]                     # clearly in
    tied = [5, 9, 17, 22, 35, 38]               # all round to 2.0
    s[tied] = 2.0 + np.array([1, 6, 2, 5, 7, 3]) * 2.0 ** -12
    sel = oracle.topk_bf16(s[None, :], None, 1, k)[0]
    assert list(sel) == [3, 5, 9, 17, 22, 30]   # the four lowest tied indices
    exact = oracle.topk(s[None, :], None, 1, k)[0]
    assert list(exact) == [3, 9, 22, 30, 35, 38]  # exact order takes the largest offsets
    # one bf16 step above the tie keeps its place
    s2 = s.copy()
    s2[38] = 2.0 + 2.0 ** -6
    assert list(oracle.topk_bf16(s2[None, :], None, 1, k)[0]) == [3, 5, 9, 17, 30, 38]
