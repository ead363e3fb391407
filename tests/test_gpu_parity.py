"""GPU parity of the HIP path (through the C ABI) against the CPU oracle,
at sizes the oracle finishes in seconds that still span several tiles and a
ragged tail.  Indices must match bit-exactly; attention outputs within
1e-2 absolute + 2e-2 relative (bf16 outputs)."""
import dataclasses
import math
import sys

import numpy as np
import pytest
import torch

import compressed_sparse_attention_02_amd as csa
import csa2_gen as G
from _ref import assert_close_bf16, npy, oracle_attend, oracle_scores, oracle_topk, u16

pytestmark = pytest.mark.gpu
DEV = "cuda"

SMALL = {
    "tiny_decode": dict(B=1, N=2048),
    "ragged_decode": dict(B=3, N=1000),
    "few_entries": dict(B=2, N=300),
    "spec_decode_qps2": dict(B=2, N=1500, q_per_seq=2),
    "qps3": dict(B=2, N=777, q_per_seq=3),
    "qps5_ratio2": dict(B=1, N=2501, q_per_seq=5, ratio=2),
    "prefill_small": dict(B=1, N=998, q_per_seq=96, ratio=2, prefix=1900),
    "mid_rows": dict(B=2, N=20000),        # row regime with a finite floor (more than 512 tiles)
    "large_rows": dict(B=2, N=40000),
    "large_rows_ragged": dict(B=2, N=40001),
    "large_qps3": dict(B=2, N=40003, q_per_seq=3),
    "prefill_large": dict(B=1, N=37500, q_per_seq=16, ratio=2, prefix=74984),
}
# rows past CSA2_TOPK_ROW_MAX: with a score matrix the tile regime reads candidate scores from it
LARGE = [n for n, v in SMALL.items() if v["N"] > csa.TOPK_ROW_MAX]


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


_cases = {}


def case(name):
    if name not in _cases:
        _cases[name] = G.make_case(name, **SMALL[name], seed=11, device=DEV)
    return _cases[name]


def run_index(c, want_scores=True):
    return csa.csa2_index(c.q_idx.view(torch.bfloat16), c.w_idx, c.k_idx.view(torch.bfloat16), c.q_pos, c.ratio,
                          c.q_per_seq, want_scores=want_scores)


def run_topk(c, ix, path="tiles", workspace=None):
    """path "rows": scores given (one-pass LDS selection when N <= 36864); "tiles": no score
    matrix, selection from tile maxima and the keys; "tiles_scores" (N > 36864): the tile
    regime with the score matrix, candidate tiles' scores read from it."""
    return csa.csa2_topk(ix.scores if path in ("rows", "tiles_scores") else None, ix.tile_max, ix.stats,
                         c.q_idx.view(torch.bfloat16), c.w_idx, c.k_idx.view(torch.bfloat16), c.q_pos, c.ratio,
                         c.q_per_seq, workspace=workspace)


def G_nvis(c, t):
    p = int(c.q_pos[t])
    return max(0, min(c.N, (p + 1) // c.ratio))


@pytest.mark.parametrize("name", list(SMALL))
def test_index_scores_within_bound(name):
    log(f"[index] {name}")
    c = case(name)
    ix = run_index(c)
    ix2 = run_index(c, want_scores=False)
    torch.cuda.synchronize()
    # the tile maxima (padding slots excluded) and the summary do not depend on whether scores
    # are written; the scan leaves the summary header zero
    nt = -(-c.N // 16)
    tm = npy(ix.tile_max)
    assert np.array_equal(tm[:, :nt], npy(ix2.tile_max)[:, :nt]) and np.array_equal(npy(ix.stats), npy(ix2.stats))
    assert np.all(npy(ix.header) == 0)
    # eps and the floor come from the selection: the tile regime's (on ix2) and the row
    # regime's eps (on ix, N <= 36864) must both bound the error
    run_topk(c, ix2, "tiles")
    run_topk(c, ix, "rows")
    torch.cuda.synchronize()
    assert np.all(npy(ix2.header)[:, 2:] == 0) and np.all(npy(ix.header)[:, 2:] == 0)
    ref = oracle_scores(c, range(c.T))
    s, e, fl = npy(ix.scores), npy(ix2.err_bound), npy(ix2.floor)
    e_rows = npy(ix.err_bound) if c.N <= csa.TOPK_ROW_MAX else e
    pad = np.full((c.T, nt * 16 - c.N), -np.inf, np.float32)
    assert np.array_equal(tm[:, :nt], np.concatenate([s, pad], axis=1).reshape(c.T, nt, 16).max(axis=2))
    worst = 0.0
    for t in range(c.T):
        nv = G_nvis(c, t)
        assert np.all(np.isneginf(s[t, nv:])), "entries beyond visibility must be -inf"
        err = np.abs(s[t, :nv].astype(np.float64) - ref[t][:nv])
        assert np.all(err <= e[t]), f"t={t}: max err {err.max()} > eps {e[t]}"
        assert np.all(err <= e_rows[t]), f"t={t}: max err {err.max()} > row-regime eps {e_rows[t]}"
        # the floor: at least 512 visible fp32 scores reach it (-inf if fewer than 512 non-empty tiles)
        if -(-nv // 16) >= 512:
            assert np.isfinite(fl[t]) and np.count_nonzero(s[t, :nv] >= fl[t]) >= 512
            # and it is useful: no more than 4 x 512 entries reach it at these sizes
            assert np.count_nonzero(s[t, :nv] >= fl[t]) <= 2048, np.count_nonzero(s[t, :nv] >= fl[t])
        else:
            assert np.isneginf(fl[t])
        if nv:
            worst = max(worst, float(err.max() / e[t]))
            # the bound must stay small next to the scores, or the candidate set explodes
            assert e[t] < 2e-3 * np.abs(ref[t][:nv]).max()
    log(f"  max |fp32 - fp64| / eps = {worst:.2e}")


@pytest.mark.parametrize("path", ["rows", "tiles", "tiles_scores"])
@pytest.mark.parametrize("name", list(SMALL))
def test_topk_bit_exact(name, path):
    if path == "tiles_scores" and name not in LARGE:
        pytest.skip("rows within CSA2_TOPK_ROW_MAX: a score matrix selects in the row regime (path rows)")
    log(f"[topk] {name} ({path})")
    c = case(name)
    ix = run_index(c, want_scores=(path != "tiles"))
    idx = run_topk(c, ix, path)
    torch.cuda.synchronize()
    assert np.all(npy(ix.header)[:, 2:] == 0), "csa2_topk must leave its counters zero"
    ref = oracle_topk(c, oracle_scores(c, range(c.T)))
    got = npy(idx)
    for t in range(c.T):
        assert np.array_equal(got[t], ref[t]), f"t={t}: {np.setdiff1d(got[t], ref[t])[:8]} vs {np.setdiff1d(ref[t], got[t])[:8]}"


def test_topk_streaming_fallback_matches():
    # a workspace with no candidate capacity forces the exact streaming path of the tile regime
    log("[topk] streaming fallback")
    c = case("large_rows_ragged")
    ix = run_index(c, want_scores=False)
    ws = torch.empty(csa.topk_min_workspace_bytes(c.T, c.N), dtype=torch.uint8, device=DEV)
    idx = run_topk(c, ix, "tiles", workspace=ws)
    torch.cuda.synchronize()
    ref = oracle_topk(c, oracle_scores(c, range(c.T)))
    for t in range(c.T):
        assert np.array_equal(npy(idx)[t], ref[t])


@pytest.mark.parametrize("path", ["rows", "tiles", "tiles_scores"])
@pytest.mark.parametrize("mode", ["all_equal", "all_equal_overflow", "all_equal_mid", "all_equal_large", "tie_block",
                                  "tie_block_mid", "tie_block_large"])
def test_topk_planted_ties(mode, path):
    if path == "tiles_scores" and not mode.endswith("_large"):
        pytest.skip("rows within CSA2_TOPK_ROW_MAX: a score matrix selects in the row regime (path rows)")
    log(f"[topk] ties {mode} ({path})")
    N = {"all_equal_overflow": 3000, "all_equal_mid": 20000, "all_equal_large": 40000, "tie_block_mid": 20000,
         "tie_block_large": 40000}.get(mode, 2048)
    c = G.make_case("ties", B=1, N=N, seed=5, device=DEV, with_kv=False)
    if mode.startswith("all_equal"):
        c.k_idx[:] = c.k_idx[0, 7]                       # every key identical: lowest 512 indices win
    else:
        # a block of identical keys whose score sits at the selection boundary
        sc = oracle_scores(c, [0])[0]
        order = np.argsort(-sc, kind="stable")
        src = int(order[500])
        c.k_idx[0, 1000:1100] = c.k_idx[0, src]
    ix = run_index(c, want_scores=(path != "tiles"))
    idx = run_topk(c, ix, path)
    torch.cuda.synchronize()
    ref = oracle_topk(c, oracle_scores(c, [0]))
    assert np.array_equal(npy(idx)[0], ref[0])
    if mode.startswith("all_equal"):
        assert list(ref[0]) == list(range(512))


def _attend(c, idx, layer=0, sink=None, window=None, swa_end=None, lse=True):
    q = c.q[layer].view(torch.bfloat16)
    swa = c.swa[layer].view(torch.bfloat16)
    return csa.csa2_attend_fp4(q, c.kv_codes, c.kv_scales, idx, swa, c.swa_end if swa_end is None else swa_end,
                               sink, c.softmax_scale, c.q_per_seq, c.window if window is None else window,
                               want_lse=lse)


@pytest.mark.parametrize("name", list(SMALL))
def test_attend_matches_oracle(name):
    log(f"[attend] {name}")
    c = case(name)
    idx = run_topk(c, run_index(c, want_scores=False))
    out, lse = _attend(c, idx)
    torch.cuda.synchronize()
    ref = oracle_attend(c, {t: npy(idx)[t] for t in range(c.T)})
    for t in range(c.T):
        mx, mean = assert_close_bf16(out[t], ref[t][0], what=f"{name} t={t}")
        np.testing.assert_allclose(npy(lse)[t], ref[t][1], rtol=1e-4, atol=1e-4)
    log(f"  last max abs err {mx:.2e}, mean {mean:.2e}")


@pytest.mark.parametrize("variant", ["window50", "short_window_end", "sink", "padded_dup_indices", "empty"])
def test_attend_edge_cases(variant):
    log(f"[attend] edge {variant}")
    c = G.make_case("edge", B=2, N=700, q_per_seq=2, seed=3, device=DEV)
    T = c.T
    rng = np.random.default_rng(0)
    idx = np.full((T, 512), -1, np.int32)
    for t in range(T):
        n = [512, 200, 77, 512][t]
        idx[t, :n] = np.sort(rng.choice(700, size=n, replace=False))
    window, swa_end, sink = c.window, npy(c.swa_end), None
    if variant == "window50":
        window = 50
    elif variant == "short_window_end":
        swa_end = np.array([0, 1, 37, 128], np.int32)
    elif variant == "sink":
        sink = np.array(np.linspace(-3, 6, 64), np.float32)
    elif variant == "padded_dup_indices":
        idx[1, 200:300] = idx[1, 5]           # duplicates are attended as separate rows
        idx[3, ::2] = -1
    elif variant == "empty":
        idx[:] = -1
        swa_end = np.zeros(T, np.int32)
    idx_t = torch.from_numpy(idx).to(DEV)
    out, lse = _attend(c, idx_t, sink=None if sink is None else torch.from_numpy(sink).to(DEV), window=window,
                       swa_end=torch.from_numpy(np.asarray(swa_end, np.int32)).to(DEV))
    torch.cuda.synchronize()
    ref = oracle_attend(c, {t: idx[t] for t in range(T)}, sink=sink, window=window, swa_end=swa_end)
    for t in range(T):
        assert_close_bf16(out[t], ref[t][0], what=f"{variant} t={t}")
        r = ref[t][1]
        g = npy(lse)[t]
        if variant == "empty":
            assert np.all(np.isneginf(g)) and np.all(npy(out[t].float()) == 0)
        else:
            np.testing.assert_allclose(g, r, rtol=1e-4, atol=1e-4)


@pytest.mark.parametrize("T_q", [1, 8, 64, 300])
def test_attend_split_plans(T_q):
    # different T choose different split-K plans (many partials + combine, or one item per query)
    log(f"[attend] split plan T={T_q}")
    c = G.make_case("split", B=T_q, N=600, seed=9, device=DEV)
    idx = run_topk(c, run_index(c, want_scores=False))
    out, lse = _attend(c, idx)
    torch.cuda.synchronize()
    ts = sorted(set([0, T_q // 2, T_q - 1]))
    ref = oracle_attend(c, {t: npy(idx)[t] for t in ts})
    for t in ts:
        assert_close_bf16(out[t], ref[t][0], what=f"T={T_q} t={t}")


# 3 sequences x 3 layers: 20 single-chunk work items per query-layer;
# 48 sequences x 3 layers: 3 work items of up to 7 chunks (eight-wave blocks both)
@pytest.mark.parametrize("B", [3, 48])
def test_reuse_layers_match_oracle_and_attend(B):
    log(f"[reuse] 3 layers, {B} sequences")
    c = G.make_case("reuse", B=B, N=1200, n_layers=4, seed=21, device=DEV)
    idx = run_topk(c, run_index(c, want_scores=False))
    full = _attend(c, idx, layer=0, lse=False)
    q = c.q[1:].view(torch.bfloat16).contiguous()
    swa = c.swa[1:].view(torch.bfloat16).contiguous()
    sink = torch.linspace(-1, 1, 3 * 64, device=DEV, dtype=torch.float32).view(3, 64)
    out, lse = csa.csa2_reuse_attend(q, c.kv_codes, c.kv_scales, idx, swa, c.swa_end, sink, c.softmax_scale,
                                     c.q_per_seq, c.window, want_lse=True)
    # Reuse with one layer and the Full layer's query reproduces the Full output exactly
    one = csa.csa2_reuse_attend(c.q[:1].view(torch.bfloat16).contiguous(), c.kv_codes, c.kv_scales, idx,
                                c.swa[:1].view(torch.bfloat16).contiguous(), c.swa_end, None, c.softmax_scale,
                                c.q_per_seq, c.window)
    torch.cuda.synchronize()
    assert torch.equal(one[0], full)
    idx_np = npy(idx)
    for l in range(3):
        ref = oracle_attend(c, {t: idx_np[t] for t in range(c.T)}, layer=l + 1, sink=npy(sink[l]))
        for t in range(c.T):
            assert_close_bf16(out[l, t], ref[t][0], what=f"layer {l} t={t}")
            np.testing.assert_allclose(npy(lse[l, t]), ref[t][1], rtol=1e-4, atol=1e-4)


def test_pipeline_is_deterministic():
    log("[determinism]")
    c = case("large_rows_ragged")
    a = run_index(c)
    a_i = run_topk(c, a, "tiles")
    a_o = _attend(c, a_i, lse=False)
    b = run_index(c)
    b_i = run_topk(c, b, "tiles")
    b_o = _attend(c, b_i, lse=False)
    torch.cuda.synchronize()
    assert torch.equal(a.scores, b.scores) and torch.equal(a.stats, b.stats)
    assert torch.equal(a.tile_max[:, :-(-c.N // 16)], b.tile_max[:, :-(-c.N // 16)])
    assert torch.equal(a_i, b_i) and torch.equal(a_o, b_o)


def test_generator_is_device_independent():
    log("[generator] cpu == gpu")
    for stream in (G.ST_KIDX, G.ST_KV, G.ST_Q):
        a = G.normal_bf16(0, stream, 12345, 70000, "cpu")
        b = G.normal_bf16(0, stream, 12345, 70000, DEV).cpu()
        assert torch.equal(a, b)
    x = G.normal_bf16(0, G.ST_KV, 0, 512 * 64, "cpu").view(64, 512)
    ca, sa = G.mxfp4_quantize(x)
    cb, sb = G.mxfp4_quantize(x.to(DEV))
    assert torch.equal(ca, cb.cpu()) and torch.equal(sa, sb.cpu())
    assert torch.equal(G.uniform_f32(0, G.ST_W, 0, 5000, "cpu"), G.uniform_f32(0, G.ST_W, 0, 5000, DEV).cpu())


def test_bound_calls_replay_the_wrappers():
    """bind(): the recorded launches reproduce the wrapper calls bit for bit, read the bound
    tensors' current contents on every call, and keep the storage they allocated alive."""
    log("[bind] index -> topk -> attend, bound vs wrapped")
    c = case("large_rows_ragged")
    bf = torch.bfloat16
    q_idx = c.q_idx.view(bf).clone()
    ix = csa.bind(csa.csa2_index, q_idx, c.w_idx, c.k_idx.view(bf), c.q_pos, c.ratio, c.q_per_seq,
                  want_scores=False)
    tk = csa.bind(csa.csa2_topk, None, ix.result.tile_max, ix.result.stats, q_idx, c.w_idx, c.k_idx.view(bf),
                  c.q_pos, c.ratio, c.q_per_seq)
    at = csa.bind(csa.csa2_attend_fp4, c.q[0].view(bf), c.kv_codes, c.kv_scales, tk.result, c.swa[0].view(bf),
                  c.swa_end, None, c.softmax_scale, c.q_per_seq, 128)
    assert len(ix._calls) == 1 and ix._calls[0][2] == "csa2_index"
    for round_ in range(2):
        if round_ == 1:  # new query contents in the same storage
            q_idx.copy_(G.normal_bf16(3, G.ST_QIDX, 0, q_idx.numel(), DEV).view(q_idx.shape).view(bf))
        ix(), tk(), at()
        w_ix = run_index(Ccase(c, q_idx), want_scores=False)
        w_i = csa.csa2_topk(None, w_ix.tile_max, w_ix.stats, q_idx, c.w_idx, c.k_idx.view(bf), c.q_pos, c.ratio,
                            c.q_per_seq)
        w_o = csa.csa2_attend_fp4(c.q[0].view(bf), c.kv_codes, c.kv_scales, w_i, c.swa[0].view(bf), c.swa_end,
                                  None, c.softmax_scale, c.q_per_seq, 128)
        torch.cuda.synchronize()
        assert torch.equal(tk.result, w_i), f"round {round_}: bound indices differ"
        assert torch.equal(at.result, w_o), f"round {round_}: bound attention differs"
    cc = Ccase(c, q_idx)
    ref = oracle_topk(cc, oracle_scores(cc, range(c.T)))
    for t in range(c.T):
        assert np.array_equal(npy(tk.result[t]), ref[t]), f"t={t}: bound indices differ from the oracle"


def Ccase(c, q_idx):
    """Case c with another indexer query (same storage layout)."""
    return dataclasses.replace(c, q_idx=q_idx.view(c.q_idx.dtype))


def test_step_graph_replays_match_eager():
    """The decode step (scan -> top-k from tile maxima -> attention -> three Reuse layers)
    captured in a HIP graph: every replay, with eager work and synchronisations between
    replays, reproduces the eager outputs bit for bit (the library records no memset and
    no host synchronisation, and resets its counters in-kernel)."""
    log("[graph] step capture and replays")
    c = G.make_case("graph", B=2, N=40001, n_layers=4, seed=11, device=DEV)
    bf = torch.bfloat16
    T, N = c.T, c.N
    tile_max = torch.empty((T, csa.tile_max_ld(N)), dtype=torch.float32, device=DEV)
    stats = torch.empty(csa.index_stats_bytes(T, c.q_per_seq, N) // 4, dtype=torch.int32, device=DEV)
    idx = torch.empty((T, 512), dtype=torch.int32, device=DEV)
    out = torch.empty((T, 64, 512), dtype=bf, device=DEV)
    out_re = torch.empty((c.n_layers - 1, T, 64, 512), dtype=bf, device=DEV)
    ws_t = torch.empty(csa.topk_workspace_bytes(T, N), dtype=torch.uint8, device=DEV)
    ws_a = torch.empty(max(1, csa.attend_workspace_bytes(T)), dtype=torch.uint8, device=DEV)
    ws_r = torch.empty(max(1, csa.attend_workspace_bytes(T, n_layers=c.n_layers - 1)), dtype=torch.uint8, device=DEV)
    q_re = c.q[1:].view(bf).contiguous()
    swa_re = c.swa[1:].view(bf).contiguous()

    def step():
        csa.csa2_index(c.q_idx.view(bf), c.w_idx, c.k_idx.view(bf), c.q_pos, c.ratio, c.q_per_seq,
                       want_scores=False, tile_max=tile_max, stats=stats)
        csa.csa2_topk(None, tile_max, stats, c.q_idx.view(bf), c.w_idx, c.k_idx.view(bf), c.q_pos, c.ratio,
                      c.q_per_seq, indices=idx, workspace=ws_t)
        csa.csa2_attend_fp4(c.q[0].view(bf), c.kv_codes, c.kv_scales, idx, c.swa[0].view(bf), c.swa_end, None,
                            c.softmax_scale, c.q_per_seq, 128, out=out, workspace=ws_a)
        csa.csa2_reuse_attend(q_re, c.kv_codes, c.kv_scales, idx, swa_re, c.swa_end, None, c.softmax_scale,
                              c.q_per_seq, 128, out=out_re, workspace=ws_r)

    step()
    torch.cuda.synchronize()
    ref = idx.clone(), out.clone(), out_re.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for r in range(4):
        idx.fill_(-7), out.zero_(), out_re.zero_(), stats.fill_(123)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, ref[0]), f"replay {r}: indices differ"
        assert torch.equal(out, ref[1]) and torch.equal(out_re, ref[2]), f"replay {r}: attention differs"
        step()  # eager work between replays
        torch.cuda.synchronize()
    ref_idx = oracle_topk(c, oracle_scores(c, range(T)))
    for t in range(T):
        assert np.array_equal(npy(idx[t]), ref_idx[t])
