"""GPU parity of csa2_attend_ex — the report's main-KV format (E2M1 + E4M3 per 16),
FP8 window rows and the fused inverse RoPE of the output — against the CPU
oracle, through the C ABI; outputs within 1e-2 absolute + 2e-2 relative (bf16),
lse within 1e-4.  Both the split-K path (merged by the combine kernel) and the
single-work-item path (written by the attention kernel) are covered."""
import sys

import numpy as np
import pytest
import torch

import compressed_sparse_attention_02_amd as csa
import csa2_gen as G
import oracle
from _ref import assert_close_bf16, npy, oracle_scores, oracle_topk, u16

pytestmark = pytest.mark.gpu
DEV = "cuda"
BF = torch.bfloat16

CASES = {
    "ragged_decode": dict(B=3, N=1000, n_layers=3),
    "prefill_wide": dict(B=1, N=1512, q_per_seq=1024, ratio=2, prefix=2000),  # 1024 queries: one work item each
}


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


_cases = {}


def case(name):
    if name not in _cases:
        c = G.make_case(name, **CASES[name], seed=41, device=DEV)
        c.extra["nv"] = G.kv_e4m3_16(c)
        c.extra["fp8"] = G.window_fp8(c)
        c.extra["ts"] = list(range(c.T)) if c.T <= 8 else [0, 1, 511, 1022, 1023]
        if c.T <= 8:
            ref = oracle_topk(c, oracle_scores(c, range(c.T)))
            idx = torch.from_numpy(np.stack([ref[t] for t in range(c.T)])).to(DEV)
        else:
            # every query's selection from the GPU path (bit-exact against the oracle elsewhere);
            # the oracle attends over the same lists
            bf = (c.q_idx.view(BF), c.w_idx, c.k_idx.view(BF), c.q_pos, c.ratio, c.q_per_seq)
            ix = csa.csa2_index(*bf)
            idx = csa.csa2_topk(ix.scores, ix.tile_max, ix.stats, *bf)
        c.extra["idx"] = idx.contiguous()
        _cases[name] = c
    return _cases[name]


def run_gpu(c, kvf, swf, rope, layer0=0, n_layers=1, sink=None):
    codes, scales = (c.kv_codes, c.kv_scales) if kvf == csa.KV_MXFP4 else c.extra["nv"]
    q = c.q[layer0:layer0 + n_layers].view(BF)
    q = q[0] if n_layers == 1 else q.contiguous()
    kw = {}
    if swf == csa.SWA_BF16:
        w = c.swa[layer0:layer0 + n_layers].view(BF)
        kw["swa"] = w[0] if n_layers == 1 else w.contiguous()
    else:
        f, r, s = [x[layer0:layer0 + n_layers] for x in c.extra["fp8"]]
        pick = (lambda x: x[0]) if n_layers == 1 else (lambda x: x.contiguous())
        kw.update(swa_fp8=pick(f), swa_rope=pick(r).view(BF), swa_scales=pick(s))
    return csa.csa2_attend_ex(q, codes, scales, c.extra["idx"], c.swa_end, sink, c.softmax_scale, c.q_per_seq, c.window,
                              kv_format=kvf, rope_pos=c.q_pos if rope else None, want_lse=True, **kw)


def run_oracle(c, kvf, swf, rope, layer, ts, sink=None):
    codes, scales = (c.kv_codes, c.kv_scales) if kvf == csa.KV_MXFP4 else c.extra["nv"]
    res = {}
    for t in ts:
        b = t // c.q_per_seq
        kw = {}
        if swf == csa.SWA_BF16:
            kw["swa"] = u16(c.swa[layer, b:b + 1])
        else:
            f, r, s = c.extra["fp8"]
            kw.update(swa_fp8=npy(f[layer, b:b + 1]), swa_rope=u16(r[layer, b:b + 1]), swa_scales=npy(s[layer, b:b + 1]))
        o, l = oracle.attend_ex(u16(c.q[layer, t:t + 1]), npy(codes[b:b + 1]), npy(scales[b:b + 1]),
                                npy(c.extra["idx"][t:t + 1]), npy(c.swa_end[t:t + 1]), sink, c.softmax_scale, 1,
                                c.window, kv_format=kvf, rope_pos=npy(c.q_pos[t:t + 1]) if rope else None, **kw)
        res[t] = (o[0], l[0])
    return res


@pytest.mark.parametrize("rope", [False, True])
@pytest.mark.parametrize("swf", [0, 1])
@pytest.mark.parametrize("kvf", [0, 1])
@pytest.mark.parametrize("name", list(CASES))
def test_attend_ex_matches_oracle(name, kvf, swf, rope):
    log(f"[attend_ex] {name} kv={kvf} swa={swf} rope={rope}")
    c = case(name)
    out, lse = run_gpu(c, kvf, swf, rope)
    torch.cuda.synchronize()
    ref = run_oracle(c, kvf, swf, rope, 0, c.extra["ts"])
    for t, (o, l) in ref.items():
        assert_close_bf16(out[t], o, what=f"{name} t={t}")
        assert np.allclose(npy(lse[t]), l, atol=1e-4, rtol=1e-5)


def test_attend_ex_default_options_equal_attend_fp4():
    c = case("ragged_decode")
    out = run_gpu(c, 0, 0, False)[0]
    ref = csa.csa2_attend_fp4(c.q[0].view(BF), c.kv_codes, c.kv_scales, c.extra["idx"], c.swa[0].view(BF), c.swa_end,
                              None, c.softmax_scale, c.q_per_seq, c.window)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


def test_attend_ex_reuse_layers_with_sink_and_rope():
    # three layers over one selection (Reuse), the report's KV format, FP8 windows, a sink
    # per layer and the output rotation
    log("[attend_ex] reuse x3, sink, E4M3 KV, FP8 window, rope")
    c = case("ragged_decode")
    sink = G.uniform_f32(5, 7, 0, 3 * 64, DEV).view(3, 64) * 4 - 2
    out, lse = run_gpu(c, 1, 1, True, layer0=0, n_layers=3, sink=sink.contiguous())
    torch.cuda.synchronize()
    for l in range(3):
        ref = run_oracle(c, 1, 1, True, l, c.extra["ts"], sink=npy(sink[l]).astype(np.float64))
        for t, (o, lr) in ref.items():
            assert_close_bf16(out[l, t], o, what=f"layer {l} t={t}")
            assert np.allclose(npy(lse[l, t]), lr, atol=1e-4, rtol=1e-5)


# Windows that end before the window length (the first tokens of a sequence: rows
# [max(0, e - 128), e), e = 0 an empty window) and fewer than k visible entries (-1
# slots in every chunk past the last entry), in every format: "short_split" runs the
# eight-wave kernel with split work items (three layers of four queries, some items
# starting in the window chunks), "short_wide" the one-item-per-query launch.
SHORT = {
    "short_split": dict(B=4, N=300, n_layers=3),
    "short_wide": dict(B=1, N=300, q_per_seq=256),
}
SHORT_ENDS = [0, 1, 31, 32, 33, 64, 100, 127, 128]


@pytest.mark.parametrize("swf", [0, 1])
@pytest.mark.parametrize("kvf", [0, 1])
@pytest.mark.parametrize("name", list(SHORT))
def test_attend_ex_short_windows_and_masked_rows(name, kvf, swf):
    log(f"[attend_ex] {name} kv={kvf} swa={swf}")
    c = G.make_case(name, **SHORT[name], seed=43, device=DEV)
    c.extra["nv"] = G.kv_e4m3_16(c)
    c.extra["fp8"] = G.window_fp8(c)
    ends = torch.tensor(SHORT_ENDS, dtype=torch.int32)
    c.swa_end = ends[torch.arange(c.T) % len(SHORT_ENDS)].to(DEV).contiguous()
    # N < k: every query selects all N entries (ascending), the rest of its slots -1
    idx = torch.full((c.T, c.k), -1, dtype=torch.int32)
    idx[:, :c.N] = torch.arange(c.N, dtype=torch.int32)
    c.extra["idx"] = idx.to(DEV).contiguous()
    L = c.n_layers
    out, lse = run_gpu(c, kvf, swf, False, layer0=0, n_layers=L)
    torch.cuda.synchronize()
    if L == 1:
        out, lse = out[None], lse[None]
    ts = list(range(c.T)) if c.T <= 16 else list(range(12)) + [100, 200, 255]
    for l in range(L):
        ref = run_oracle(c, kvf, swf, False, l, ts)
        for t, (o, lr) in ref.items():
            assert_close_bf16(out[l, t], o, what=f"{name} layer {l} t={t} end={int(c.swa_end[t])}")
            assert np.allclose(npy(lse[l, t]), lr, atol=1e-4, rtol=1e-5)
