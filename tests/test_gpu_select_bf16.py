"""GPU parity of the BF16 selector (csa2_topk_ex / csa2_topk_mxfp4_ex with
CSA2_SELECT_BF16) against the CPU oracle's topk_bf16: every exact score rounded
to the nearest bf16 value, then (value desc, index asc).  Indices bit-exact, in
both selection regimes (score rows in LDS; tile maxima and keys), through the
streaming fallback, with planted near-ties that only the rounding makes equal,
and with MXFP4 indexer keys."""
import sys

import numpy as np
import pytest
import torch

import compressed_sparse_attention_02_amd as csa
import csa2_gen as G
import oracle
from _ref import npy, oracle_scores

pytestmark = pytest.mark.gpu
DEV = "cuda"
BF = torch.bfloat16

CASES = {
    "tiny_decode": dict(B=1, N=2048),
    "ragged_decode": dict(B=3, N=1000),
    "few_entries": dict(B=2, N=300),
    "qps5_ratio2": dict(B=1, N=2501, q_per_seq=5, ratio=2),
    "prefill_small": dict(B=1, N=998, q_per_seq=96, ratio=2, prefix=1900),
    "large_rows": dict(B=2, N=40000),
    "long_rows_ragged": dict(B=2, N=100003),
}


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


_cases = {}


def case(name):
    if name not in _cases:
        _cases[name] = G.make_case(name, **CASES[name], seed=17, device=DEV, with_kv=False)
    return _cases[name]


def select(c, path, workspace=None, mode=csa.SELECT_BF16):
    ix = csa.csa2_index(c.q_idx.view(BF), c.w_idx, c.k_idx.view(BF), c.q_pos, c.ratio, c.q_per_seq,
                        want_scores=(path == "rows"))
    return csa.csa2_topk(ix.scores if path == "rows" else None, ix.tile_max, ix.stats, c.q_idx.view(BF), c.w_idx,
                         c.k_idx.view(BF), c.q_pos, c.ratio, c.q_per_seq, workspace=workspace, select=mode)


def oracle_bf16(c, scores_by_t):
    return {t: oracle.topk_bf16(s[None, :], npy(c.q_pos[t:t + 1]), c.ratio, c.k)[0] for t, s in scores_by_t.items()}


def check(got, ref, what):
    g = npy(got)
    for t, r in ref.items():
        assert np.array_equal(g[t], r), f"{what} t={t}: {np.setdiff1d(g[t], r)[:8]} vs {np.setdiff1d(r, g[t])[:8]}"


@pytest.mark.parametrize("path", ["rows", "tiles"])
@pytest.mark.parametrize("name", list(CASES))
def test_bf16_select_bit_exact(name, path):
    log(f"[bf16 select] {name} ({path})")
    c = case(name)
    if path == "rows" and c.N > csa.TOPK_ROW_MAX:
        pytest.skip("rows longer than the row regime always take the tile regime")
    idx = select(c, path)
    torch.cuda.synchronize()
    check(idx, oracle_bf16(c, oracle_scores(c, range(c.T))), name)


def test_bf16_select_streaming_fallback():
    """No candidate capacity: the tile regime's exact streaming path, in bf16 order."""
    log("[bf16 select] streaming fallback")
    c = case("large_rows")
    ws = torch.empty(csa.topk_min_workspace_bytes(c.T, c.N), dtype=torch.uint8, device=DEV)
    idx = select(c, "tiles", workspace=ws)
    torch.cuda.synchronize()
    check(idx, oracle_bf16(c, oracle_scores(c, range(c.T))), "streaming")


@pytest.mark.parametrize("path", ["rows", "tiles"])
@pytest.mark.parametrize("N", [2048, 40000])
def test_bf16_select_planted_near_ties(N, path):
    """100 keys made from the key ranked near the cut by changing one channel by one bf16 step:
    their exact scores differ, most of them round to the same bf16 value, and the lower index
    must win among those; the exact order picks differently."""
    if path == "rows" and N > csa.TOPK_ROW_MAX:
        pytest.skip("tile regime only")
    log(f"[bf16 select] near ties N={N} ({path})")
    c = G.make_case("near_ties", B=1, N=N, seed=23, device=DEV, with_kv=False)
    sc = oracle_scores(c, [0])[0]
    src = int(np.argsort(-sc, kind="stable")[480])
    rows = c.k_idx[0, src].clone().repeat(100, 1)
    rng = np.random.default_rng(5)
    ch = torch.from_numpy(rng.integers(0, 128, 100)).to(DEV)
    step = torch.from_numpy(rng.choice([-1, 1], 100)).to(DEV).to(torch.int16)
    r = torch.arange(100, device=DEV)
    rows[r, ch] = rows[r, ch] + step  # neighbouring bf16 value of one channel
    c.k_idx[0, 1000:1100] = rows
    ref_s = oracle_scores(c, [0])
    ref = oracle_bf16(c, ref_s)
    exact = oracle.topk(ref_s[0][None, :], npy(c.q_pos[:1]), c.ratio, c.k)[0]
    assert not np.array_equal(ref[0], exact), "the planted case must separate the two orders"
    idx = select(c, path)
    idx_exact = select(c, path, mode=csa.SELECT_EXACT)
    torch.cuda.synchronize()
    check(idx, ref, "bf16")
    assert np.array_equal(npy(idx_exact)[0], exact)


@pytest.mark.parametrize("path", ["rows", "tiles"])
@pytest.mark.parametrize("name", ["ragged_decode", "large_rows"])
def test_bf16_select_mxfp4_keys(name, path):
    log(f"[bf16 select] MXFP4 keys {name} ({path})")
    c = case(name)
    qc, qs, kc, ks = G.mx_indexer(c)
    ix = csa.csa2_index_mxfp4(qc, qs, c.w_idx, kc, ks, c.q_pos, c.ratio, c.q_per_seq, want_scores=(path == "rows"))
    idx = csa.csa2_topk_mxfp4(ix.scores if path == "rows" else None, ix.tile_max, ix.stats, c.w_idx, kc, ks,
                              c.q_pos, c.ratio, c.q_per_seq, select=csa.SELECT_BF16)
    torch.cuda.synchronize()
    qcn, qsn, kcn, ksn = npy(qc), npy(qs), npy(kc), npy(ks)
    ref_s = {}
    for t in range(c.T):
        b = t // c.q_per_seq
        ref_s[t] = oracle.index_mx(qcn[t:t + 1], qsn[t:t + 1], npy(c.w_idx[t:t + 1]), kcn[b:b + 1], ksn[b:b + 1],
                                   npy(c.q_pos[t:t + 1]), c.ratio, 1)[0]
    check(idx, oracle_bf16(c, ref_s), "mxfp4")
