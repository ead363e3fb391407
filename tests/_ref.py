"""Oracle-side helpers for the GPU parity tests (CPU, numpy)."""
import numpy as np
import torch

import csa2_gen as G
import oracle


def u16(t):
    return np.ascontiguousarray(t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16))


def npy(t):
    return np.ascontiguousarray(t.detach().cpu().numpy())


def oracle_scores(c, ts):
    """fp64 oracle scores for queries ts of case c -> {t: float64 [N]}."""
    out = {}
    for t in ts:
        b = t // c.q_per_seq
        s = oracle.index(u16(c.q_idx[t:t + 1]), npy(c.w_idx[t:t + 1]), u16(c.k_idx[b:b + 1]),
                         npy(c.q_pos[t:t + 1]), c.ratio, 1)
        out[t] = s[0]
    return out


def oracle_topk(c, scores_by_t):
    out = {}
    for t, s in scores_by_t.items():
        out[t] = oracle.topk(s[None, :], npy(c.q_pos[t:t + 1]), c.ratio, c.k)[0]
    return out


def oracle_attend(c, indices_by_t, layer=0, sink=None, window=None, swa_end=None):
    """Oracle attention of queries indices_by_t.keys() for one layer -> {t: (out [64][512], lse [64])}."""
    window = c.window if window is None else window
    swa_end = npy(c.swa_end) if swa_end is None else np.asarray(swa_end, np.int32)
    res = {}
    for t, idx in indices_by_t.items():
        b = t // c.q_per_seq
        o, l = oracle.attend(u16(c.q[layer, t:t + 1]), npy(c.kv_codes[b:b + 1]), npy(c.kv_scales[b:b + 1]),
                             np.asarray(idx, np.int32)[None, :], u16(c.swa[layer, b:b + 1]),
                             swa_end[t:t + 1], None if sink is None else np.asarray(sink, np.float64),
                             c.softmax_scale, 1, window)
        res[t] = (o[0], l[0])
    return res


def assert_close_bf16(gpu_out, ref, atol=1e-2, rtol=2e-2, what=""):
    g = gpu_out.float().cpu().numpy().astype(np.float64)
    err = np.abs(g - ref)
    bad = err > atol + rtol * np.abs(ref)
    assert not bad.any(), (f"{what}: {bad.sum()} elements out of tolerance; max abs err {err.max():.3e}, "
                           f"worst at {np.unravel_index(np.argmax(err - rtol * np.abs(ref)), err.shape)}")
    return float(err.max()), float(err.mean())
