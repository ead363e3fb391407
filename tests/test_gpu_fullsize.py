"""Full-size GPU parity on sampled queries, at the workloads' real shapes and
in the launch configuration the benchmark times.

Inputs are generated on the GPU by the seeded counter-based generator (bit-
identical to its CPU output, see test_generator_is_device_independent) and
copied to the host for the oracle.  For each sampled query the oracle scores
every visible entry in fp64, so the top-512 comparison is exact and complete;
attention is checked on the full 64 x 512 output of those queries.
"""
import sys

import numpy as np
import pytest
import torch

import compressed_sparse_attention_02_amd as csa
import csa2_gen as G
from _ref import assert_close_bf16, npy, oracle_attend, oracle_scores, oracle_topk

pytestmark = pytest.mark.gpu
DEV = "cuda"
BF = torch.bfloat16


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_full(c, layers=1, path="tiles"):
    """The benchmarked pipeline: with path "tiles" the scan writes no score matrix and the
    selection works from tile maxima and keys; with "rows" the scores are materialised and
    selected in LDS; with "scores" (rows past CSA2_TOPK_ROW_MAX, the many-query decode
    workloads) the scan writes the matrix and the tile regime reads candidate scores from it.
    Without a matrix a second scan provides the scores for the bound check."""
    bf = (c.q_idx.view(BF), c.w_idx, c.k_idx.view(BF), c.q_pos, c.ratio, c.q_per_seq)
    ix = csa.csa2_index(*bf, want_scores=(path != "tiles"))
    idx = csa.csa2_topk(ix.scores, ix.tile_max, ix.stats, *bf)
    out = csa.csa2_attend_fp4(c.q[0].view(BF), c.kv_codes, c.kv_scales, idx, c.swa[0].view(BF), c.swa_end, None,
                              c.softmax_scale, c.q_per_seq, c.window)
    re = None
    if layers > 1:
        re = csa.csa2_reuse_attend(c.q[1:].view(BF).contiguous(), c.kv_codes, c.kv_scales, idx,
                                   c.swa[1:].view(BF).contiguous(), c.swa_end, None, c.softmax_scale, c.q_per_seq,
                                   c.window)
    full = ix if path != "tiles" else csa.csa2_index(*bf)
    torch.cuda.synchronize()
    nt, h = -(-c.N // 16), c.T * csa.STATS_WORDS
    # same tile maxima and summary (past the header, which csa2_topk fills) with and without scores
    assert torch.equal(full.tile_max[:, :nt], ix.tile_max[:, :nt]) and torch.equal(full.stats[h:], ix.stats[h:])
    return full.scores, ix.err_bound, idx, out, re


def check_sampled(c, ts, layers=1, path="tiles"):
    scores, eps, idx, out, re = run_full(c, layers, path)
    log(f"  GPU path done; oracle on queries {ts}")
    ref_s = oracle_scores(c, ts)
    ref_i = oracle_topk(c, ref_s)
    s_np, e_np, i_np = npy(scores[ts]), npy(eps[ts]), npy(idx[ts])
    for j, t in enumerate(ts):
        nv = max(0, min(c.N, (int(c.q_pos[t]) + 1) // c.ratio))
        err = np.abs(s_np[j, :nv].astype(np.float64) - ref_s[t][:nv])
        assert np.all(err <= e_np[j]), f"t={t}: score error {err.max()} > eps {e_np[j]}"
        assert np.all(np.isneginf(s_np[j, nv:]))
        assert np.array_equal(i_np[j], ref_i[t]), f"t={t}: top-512 differs"
        log(f"  t={t}: n_vis={nv} max|err|/eps={err.max() / e_np[j]:.2e}, indices exact")
    ref_o = oracle_attend(c, {t: ref_i[t] for t in ts})
    for t in ts:
        mx, mean = assert_close_bf16(out[t], ref_o[t][0], what=f"{c.name} t={t}")
        log(f"  t={t}: attention max abs err {mx:.2e}")
    if re is not None:
        for l in range(layers - 1):
            ref_r = oracle_attend(c, {t: ref_i[t] for t in ts}, layer=l + 1)
            for t in ts:
                assert_close_bf16(re[l, t], ref_r[t][0], what=f"{c.name} reuse layer {l} t={t}")
        log(f"  {layers - 1} Reuse layers within tolerance")


def test_tiny_decode_all_queries():
    log("[full] tiny_decode")
    c = G.make_case("tiny_decode", **G.CONFIGS["tiny_decode"], seed=0, device=DEV)
    check_sampled(c, [0])


def test_long_decode_sampled():
    log("[full] long_decode 4 x 1M")
    c = G.make_case("long_decode", **G.CONFIGS["long_decode"], seed=0, device=DEV)
    check_sampled(c, [0, 3])


def test_batched_decode_sampled():
    log("[full] batched_decode 64 x 128K")
    c = G.make_case("batched_decode", **G.CONFIGS["batched_decode"], seed=0, device=DEV)
    check_sampled(c, [0, 37, 63])


def test_reuse_group_sampled():
    log("[full] reuse_group 32 x 256K, Full + 3 Reuse")
    c = G.make_case("reuse_group", **G.CONFIGS["reuse_group"], seed=0, device=DEV)
    check_sampled(c, [0, 31], layers=4)


def test_batched_decode_score_matrix_sampled():
    """The tile regime reading candidate scores from a score matrix, at the batched shape."""
    log("[full] batched_decode 64 x 128K, score matrix given")
    c = G.make_case("batched_decode", **G.CONFIGS["batched_decode"], seed=0, device=DEV)
    check_sampled(c, [5, 62], path="scores")


@pytest.mark.parametrize("path", ["rows", "tiles"])
def test_causal_prefill_sampled(path):
    log(f"[full] causal_prefill 4096 queries, 34816 entries, ratio 2 ({path})")
    c = G.make_case("causal_prefill", **G.CONFIGS["causal_prefill"], seed=0, device=DEV)
    check_sampled(c, [0, 1, 2047, 4094, 4095], path=path)


def check_hierarchical(c, ts):
    """Candidate pool and Reindex selection at full size: exact against the oracle on queries ts;
    Reindex with the Full query equals the Full top-512 on every query (a property at any size)."""
    import oracle
    from _ref import u16
    bf = (c.q_idx.view(BF), c.w_idx, c.k_idx.view(BF), c.q_pos, c.ratio, c.q_per_seq)
    ix = csa.csa2_index(*bf, want_scores=False)
    pool = csa.csa2_hsi_pool(ix.tile_max, ix.stats, *bf)
    full = csa.csa2_topk(None, ix.tile_max, ix.stats, *bf)
    same = csa.csa2_reindex(pool, c.q_idx.view(BF), c.w_idx, c.k_idx.view(BF), c.q_per_seq)
    q2 = G.normal_bf16(1, G.ST_QIDX, 0, c.T * csa.IDX_HEADS * csa.IDX_DIM, DEV).view(c.T, csa.IDX_HEADS,
                                                                                    csa.IDX_DIM)
    w2 = G.uniform_f32(1, G.ST_W, 0, c.T * csa.IDX_HEADS, DEV).view(c.T, csa.IDX_HEADS)
    re = csa.csa2_reindex(pool, q2.view(BF), w2, c.k_idx.view(BF), c.q_per_seq)
    torch.cuda.synchronize()
    assert torch.equal(full, same), "Reindex with the Full query must return the Full top-512"
    log(f"  GPU path done; oracle on queries {ts}")
    ref_s = oracle_scores(c, ts)
    p_np, r_np = npy(pool), npy(re)
    for t in ts:
        b = t // c.q_per_seq
        ref_p = oracle.hsi_pool(ref_s[t][None, :], npy(c.q_pos[t:t + 1]), c.ratio)[0]
        assert np.array_equal(p_np[t], ref_p), f"t={t}: pool differs"
        s2 = oracle.index(u16(q2[t:t + 1]), npy(w2[t:t + 1]), u16(c.k_idx[b:b + 1]), npy(c.q_pos[t:t + 1]),
                          c.ratio, 1)
        ref_r = oracle.reindex_topk(s2, ref_p[None, :], c.k)[0]
        assert np.array_equal(r_np[t], ref_r), f"t={t}: Reindex top-512 differs"
        log(f"  t={t}: pool of {int((ref_p >= 0).sum())} entries and Reindex top-512 exact")


def test_long_decode_hierarchical_sampled():
    log("[full] long_decode 4 x 1M: candidate pool + Reindex")
    c = G.make_case("long_decode", **G.CONFIGS["long_decode"], seed=0, device=DEV, with_kv=False)
    check_hierarchical(c, [1, 2])


def test_causal_prefill_hierarchical_sampled():
    log("[full] causal_prefill 4096 queries: candidate pool + Reindex")
    c = G.make_case("causal_prefill", **G.CONFIGS["causal_prefill"], seed=0, device=DEV, with_kv=False)
    check_hierarchical(c, [0, 2048, 4095])


def test_long_decode_mxfp4_indexer_sampled():
    # the MXFP4 indexer at the long-decode shape: scores within the bound and the exact
    # top-512 on sampled queries; attention over that selection within tolerance
    import oracle
    log("[full] long_decode 4 x 1M, MXFP4 indexer")
    c = G.make_case("long_decode", **G.CONFIGS["long_decode"], seed=0, device=DEV)
    qc, qs, kc, ks = G.mx_indexer(c)
    ix = csa.csa2_index_mxfp4(qc, qs, c.w_idx, kc, ks, c.q_pos, 1, 1, want_scores=False)
    idx = csa.csa2_topk_mxfp4(None, ix.tile_max, ix.stats, c.w_idx, kc, ks, c.q_pos, 1, 1)
    out = csa.csa2_attend_fp4(c.q[0].view(BF), c.kv_codes, c.kv_scales, idx, c.swa[0].view(BF), c.swa_end, None,
                              c.softmax_scale, 1, c.window)
    full = csa.csa2_index_mxfp4(qc, qs, c.w_idx, kc, ks, c.q_pos, 1, 1)
    torch.cuda.synchronize()
    assert torch.equal(full.tile_max, ix.tile_max)
    eps = npy(ix.err_bound)
    for t in [0, 3]:
        ref = oracle.index_mx(npy(qc[t:t + 1]), npy(qs[t:t + 1]), npy(c.w_idx[t:t + 1]), npy(kc[t:t + 1]),
                              npy(ks[t:t + 1]), npy(c.q_pos[t:t + 1]), 1, 1)
        err = np.abs(npy(full.scores[t]).astype(np.float64) - ref[0])
        assert np.all(err <= eps[t]), f"t={t}: {err.max()} > {eps[t]}"
        ref_i = oracle.topk(ref, npy(c.q_pos[t:t + 1]), 1, 512)[0]
        assert np.array_equal(npy(idx[t]), ref_i), f"t={t}: top-512 differs"
        ref_o = oracle_attend(c, {t: ref_i})
        assert_close_bf16(out[t], ref_o[t][0], what=f"mx t={t}")
        log(f"  t={t}: max|err|/eps={err.max() / eps[t]:.2e}, indices exact, attention within tolerance")


def test_long_decode_deployed_formats_sampled():
    # the report's deployed formats at the long-decode shape: E4M3/16 main KV, FP8 windows and
    # the output rotation, over the exact selection of sampled queries
    import oracle
    from _ref import u16
    log("[full] long_decode 4 x 1M, E4M3/16 KV + FP8 window + inverse RoPE")
    c = G.make_case("long_decode", **G.CONFIGS["long_decode"], seed=0, device=DEV)
    bf = (c.q_idx.view(BF), c.w_idx, c.k_idx.view(BF), c.q_pos, 1, 1)
    ix = csa.csa2_index(*bf, want_scores=False)
    idx = csa.csa2_topk(None, ix.tile_max, ix.stats, *bf)
    nc, ns = G.kv_e4m3_16(c)
    f8, rp, s8 = (x[0].contiguous() for x in G.window_fp8(c))
    out = csa.csa2_attend_ex(c.q[0].view(BF), nc, ns, idx, c.swa_end, None, c.softmax_scale, 1, c.window,
                             kv_format=csa.KV_E4M3_16, swa_fp8=f8, swa_rope=rp.view(BF), swa_scales=s8,
                             rope_pos=c.q_pos)
    torch.cuda.synchronize()
    for t in [1, 2]:
        o, _ = oracle.attend_ex(u16(c.q[0, t:t + 1]), npy(nc[t:t + 1]), npy(ns[t:t + 1]), npy(idx[t:t + 1]),
                                npy(c.swa_end[t:t + 1]), None, c.softmax_scale, 1, c.window, kv_format=1,
                                swa_fp8=npy(f8[t:t + 1]), swa_rope=u16(rp[t:t + 1]), swa_scales=npy(s8[t:t + 1]),
                                rope_pos=npy(c.q_pos[t:t + 1]))
        assert_close_bf16(out[t], o[0], what=f"deployed formats t={t}")
        log(f"  t={t}: within tolerance")
