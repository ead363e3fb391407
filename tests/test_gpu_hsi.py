"""GPU parity of the hierarchical sparse indexer's candidate pool (csa2_hsi_pool)
and the Reindex selection (csa2_reindex) against the CPU oracle, through the
C ABI.  Pools and indices are integer results and must match bit-exactly.

The Reindex layer's indexer query comes from the seeded generator under a
seed of its own; it shares the Full layer's indexer keys."""
import sys

import numpy as np
import pytest
import torch

import compressed_sparse_attention_02_amd as csa
import csa2_gen as G
import oracle
from _ref import npy, oracle_scores, oracle_topk, u16

pytestmark = pytest.mark.gpu
DEV = "cuda"
BF = torch.bfloat16

CASES = {
    "short_rows": dict(B=2, N=10000),                   # fewer than 16384 visible: the whole row
    "exactly_pool": dict(B=2, N=16384),                 # 2048 blocks: all of them
    "one_block_more": dict(B=2, N=16385),               # 2049 blocks, the last one partial
    "ragged_rows": dict(B=3, N=17001),
    "tile_maxima": dict(B=2, N=100003),                 # floor from the tile maxima
    "group_maxima": dict(B=2, N=200003),                # floor from the scan's group maxima
    "spec_qps3": dict(B=2, N=40001, q_per_seq=3),
    "prefill_straddle": dict(B=1, N=16402, q_per_seq=64, ratio=2, prefix=32740),  # n_vis 16370 .. 16402
}


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


_cases = {}


def case(name):
    if name not in _cases:
        _cases[name] = G.make_case(name, **CASES[name], seed=23, device=DEV, with_kv=False)
    return _cases[name]


def reindex_query(c, seed=1023):
    """The Reindex layer's own indexer query (seeded, same shapes as the Full layer's)."""
    q = G.normal_bf16(seed, G.ST_QIDX, 0, c.T * csa.IDX_HEADS * csa.IDX_DIM, DEV).view(c.T, csa.IDX_HEADS,
                                                                                       csa.IDX_DIM)
    w = G.uniform_f32(seed, G.ST_W, 0, c.T * csa.IDX_HEADS, DEV).view(c.T, csa.IDX_HEADS)
    return q, w


def oracle_scores_with(c, q, w, ts):
    """fp64 oracle scores of queries ts for indexer query (q, w) over c's keys -> {t: [N]}."""
    out = {}
    for t in ts:
        b = t // c.q_per_seq
        s = oracle.index(u16(q[t:t + 1]), npy(w[t:t + 1]), u16(c.k_idx[b:b + 1]), npy(c.q_pos[t:t + 1]),
                         c.ratio, 1)
        out[t] = s[0]
    return out


def oracle_pool(c, scores_by_t):
    return {t: oracle.hsi_pool(s[None, :], npy(c.q_pos[t:t + 1]), c.ratio)[0] for t, s in scores_by_t.items()}


def run_pool(c):
    bf = (c.q_idx.view(BF), c.w_idx, c.k_idx.view(BF), c.q_pos, c.ratio, c.q_per_seq)
    ix = csa.csa2_index(*bf, want_scores=False)
    pool = csa.csa2_hsi_pool(ix.tile_max, ix.stats, *bf)
    return ix, pool


def n_vis(c, t):
    return max(0, min(c.N, (int(c.q_pos[t]) + 1) // c.ratio))


@pytest.mark.parametrize("name", list(CASES))
def test_pool_bit_exact(name):
    log(f"[hsi] {name}")
    c = case(name)
    ix, pool = run_pool(c)
    torch.cuda.synchronize()
    ref = oracle_pool(c, oracle_scores(c, range(c.T)))
    got = npy(pool)
    for t in range(c.T):
        nv = n_vis(c, t)
        assert np.array_equal(got[t], ref[t]), (
            f"t={t} n_vis={nv}: {np.setdiff1d(got[t], ref[t])[:8]} vs {np.setdiff1d(ref[t], got[t])[:8]}")
        if nv <= csa.HSI_POOL:
            assert list(got[t][:nv]) == list(range(nv))
    # the summary header is the selection's to fill: the pool leaves it as the scan wrote it
    assert np.all(npy(ix.header) == 0)


@pytest.mark.parametrize("mode", ["all_equal", "tie_blocks", "planted_blocks"])
def test_pool_planted(mode):
    log(f"[hsi] planted {mode}")
    c = G.make_case("hsi_ties", B=1, N=40000, seed=7, device=DEV, with_kv=False)
    if mode == "all_equal":
        c.k_idx[:] = c.k_idx[0, 11]            # every block ties: the lowest 2048 blocks win
    elif mode == "tie_blocks":
        # a run of identical keys whose score sits at the 2048th block score: the blocks they
        # fill tie and the boundary falls inside the run
        sc = oracle_scores(c, [0])[0]
        bmax = sc.reshape(-1, 8).max(axis=1)
        src_blk = int(np.argsort(-bmax, kind="stable")[2040])
        src = src_blk * 8 + int(np.argmax(sc[src_blk * 8:src_blk * 8 + 8]))
        c.k_idx[0, 20000:20200] = c.k_idx[0, src]
    else:
        # the best key copied into scattered single entries: each of their blocks must be kept
        sc = oracle_scores(c, [0])[0]
        best = int(np.argmax(sc))
        for e in range(3, 40000, 997):
            c.k_idx[0, e] = c.k_idx[0, best]
    ix, pool = run_pool(c)
    torch.cuda.synchronize()
    ref = oracle_pool(c, oracle_scores(c, [0]))
    got = npy(pool)[0]
    assert np.array_equal(got, ref[0])
    if mode == "all_equal":
        assert list(got) == list(range(csa.HSI_POOL))
    if mode == "planted_blocks":
        assert set(range(3, 40000, 997)) <= set(got.tolist())


@pytest.mark.parametrize("name", ["short_rows", "one_block_more", "tile_maxima", "spec_qps3", "prefill_straddle"])
def test_reindex_bit_exact(name):
    log(f"[reindex] {name}")
    c = case(name)
    ix, pool = run_pool(c)
    q2, w2 = reindex_query(c)
    idx = csa.csa2_reindex(pool, q2.view(BF), w2, c.k_idx.view(BF), c.q_per_seq)
    torch.cuda.synchronize()
    ref_pool = oracle_pool(c, oracle_scores(c, range(c.T)))
    s2 = oracle_scores_with(c, q2, w2, range(c.T))
    got = npy(idx)
    for t in range(c.T):
        ref = oracle.reindex_topk(s2[t][None, :], ref_pool[t][None, :], c.k)[0]
        assert np.array_equal(got[t], ref), f"t={t}: {np.setdiff1d(got[t], ref)[:8]} vs {np.setdiff1d(ref, got[t])[:8]}"
        assert set(got[t][got[t] >= 0].tolist()) <= set(ref_pool[t][ref_pool[t] >= 0].tolist())


def test_reindex_with_full_query_is_full_topk():
    # the pool holds the Full layer's whole top-512, so a Reindex pass with the Full
    # layer's own query must return csa2_topk's selection
    log("[reindex] Full query")
    c = case("group_maxima")
    bf = (c.q_idx.view(BF), c.w_idx, c.k_idx.view(BF), c.q_pos, c.ratio, c.q_per_seq)
    ix, pool = run_pool(c)
    full = csa.csa2_topk(None, ix.tile_max, ix.stats, *bf)
    re = csa.csa2_reindex(pool, c.q_idx.view(BF), c.w_idx, c.k_idx.view(BF), c.q_per_seq)
    torch.cuda.synchronize()
    assert torch.equal(full, re)
    ref = oracle_topk(c, oracle_scores(c, [0]))
    assert np.array_equal(npy(re)[0], ref[0])


def test_reindex_small_pool_pads():
    # fewer than 512 visible entries: the Reindex selection keeps the whole pool
    log("[reindex] small pool")
    c = G.make_case("hsi_small", B=2, N=300, seed=3, device=DEV, with_kv=False)
    ix, pool = run_pool(c)
    q2, w2 = reindex_query(c)
    idx = csa.csa2_reindex(pool, q2.view(BF), w2, c.k_idx.view(BF), c.q_per_seq)
    torch.cuda.synchronize()
    got = npy(idx)
    for t in range(c.T):
        assert list(got[t][:300]) == list(range(300)) and np.all(got[t][300:] == -1)


def test_pool_and_reindex_are_deterministic():
    log("[hsi] determinism")
    c = case("ragged_rows")
    _, p1 = run_pool(c)
    _, p2 = run_pool(c)
    q2, w2 = reindex_query(c)
    r1 = csa.csa2_reindex(p1, q2.view(BF), w2, c.k_idx.view(BF), c.q_per_seq)
    r2 = csa.csa2_reindex(p2, q2.view(BF), w2, c.k_idx.view(BF), c.q_per_seq)
    torch.cuda.synchronize()
    assert torch.equal(p1, p2) and torch.equal(r1, r2)
