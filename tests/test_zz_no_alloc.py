"""csa2_reuse_attend_static, the entry point that allocates nothing, against csa2_reuse_attend
with a caller workspace, through the C ABI: bit-identical outputs and lse on two calls in a
row (the second with a smaller input), nothing allocated by the call, and the launch shape with
the largest partial workspace, which the library's static scratch must hold."""
import sys

import numpy as np
import pytest
import torch

import compressed_sparse_attention_02_amd as csa
import csa2_gen as G

pytestmark = pytest.mark.gpu
DEV = "cuda"
BF = torch.bfloat16


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def selection(c):
    ix = csa.csa2_index(c.q_idx.view(BF), c.w_idx, c.k_idx.view(BF), c.q_pos, c.ratio, c.q_per_seq,
                        want_scores=False)
    return csa.csa2_topk(None, ix.tile_max, ix.stats, c.q_idx.view(BF), c.w_idx, c.k_idx.view(BF), c.q_pos,
                         c.ratio, c.q_per_seq)


def compare(c, L, sink):
    q = c.q[:L].view(BF).contiguous()
    swa = c.swa[:L].view(BF).contiguous()
    idx = selection(c)
    ref, ref_lse = csa.csa2_reuse_attend(q, c.kv_codes, c.kv_scales, idx, swa, c.swa_end, sink, c.softmax_scale,
                                         c.q_per_seq, c.window, want_lse=True)
    out = torch.full_like(ref, 7)
    lse = torch.full_like(ref_lse, 7)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    csa.csa2_reuse_attend_static(q, c.kv_codes, c.kv_scales, idx, swa, c.swa_end, sink, c.softmax_scale,
                                 c.q_per_seq, c.window, out=out, lse=lse)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before, "the static entry point allocated through torch"
    assert torch.equal(out, ref), f"outputs differ: {int((out != ref).sum())} elements"
    assert torch.equal(lse, ref_lse)
    return out


def test_static_matches_workspace_call_twice():
    # first call: 6 sequences x 3 layers with a sink (split over 10 work items per query-layer)
    log("[no-alloc] call 1: T=6, L=3, sink")
    c1 = G.make_case("noalloc1", B=6, N=3000, n_layers=3, seed=31, device=DEV)
    sink = torch.linspace(-2, 2, 3 * 64, device=DEV, dtype=torch.float32).view(3, 64)
    a = compare(c1, 3, sink)
    # second call on the same array, a smaller input: 2 sequences, one layer, no sink
    log("[no-alloc] call 2: T=2, L=1")
    c2 = G.make_case("noalloc2", B=2, N=1200, n_layers=1, seed=32, device=DEV)
    compare(c2, 1, None)
    assert a.abs().sum() > 0


def test_static_largest_split():
    # the launch shape with the largest partial workspace (160 queries, a 33-row window: 18
    # chunks over 3 work items, 30.2 MiB), which the static array must hold
    T, window = 160, 33
    need = csa.attend_workspace_bytes(T, window=window)
    assert 30 * 2 ** 20 < need <= csa.STATIC_SCRATCH_BYTES
    log(f"[no-alloc] T={T}, window={window}: {need} bytes of partials")
    c = G.make_case("noalloc3", B=T, N=600, window=window, n_layers=1, seed=33, device=DEV)
    compare(c, 1, None)
