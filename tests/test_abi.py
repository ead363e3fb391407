"""C-ABI library checks that need no GPU: it loads, exports every declared
entry point, and rejects bad arguments on the host before launching anything."""
import ctypes
import os
import re

import pytest

import compressed_sparse_attention_02_amd as csa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa2.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(csa2_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    return csa.lib()


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert {"csa2_index", "csa2_topk", "csa2_attend_fp4", "csa2_reuse_attend", "csa2_hsi_pool",
            "csa2_reindex", "csa2_index_mxfp4", "csa2_topk_mxfp4", "csa2_hsi_pool_mxfp4",
            "csa2_reindex_mxfp4", "csa2_attend_ex", "csa2_kv_write", "csa2_topk_ex",
            "csa2_topk_mxfp4_ex"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings_and_version(L):
    assert L.csa2_status_string(0) == b"CSA2_OK"
    assert L.csa2_status_string(3) == b"CSA2_ERR_WORKSPACE"
    assert L.csa2_status_string(99) == b"CSA2_ERR_UNKNOWN"
    assert b"gfx950" in L.csa2_version()


def test_workspace_queries(L):
    # the summary: a 4-word header per query, group maxima and norm partials
    assert csa.index_stats_bytes(4, 1, 1 << 20) >= 4 * 4 * 4 + 4 * 4096 * 4
    assert csa.index_stats_bytes(4, 3, 100) == 0              # T not a multiple of q_per_seq
    assert csa.index_stats_bytes(1, 1, 1 << 31) == 0          # N beyond 2^31 - 1
    assert csa.topk_workspace_bytes(4, 1 << 20) >= csa.topk_min_workspace_bytes(4, 1 << 20) > 0
    assert csa.topk_workspace_bytes(4, 1 << 20, 256) == 0      # only k = 512
    assert csa.topk_workspace_bytes(4, 30000) > 0              # tile regime needs one even for short rows
    assert csa.attend_workspace_bytes(4096) == 0               # one work item per query: no partials
    assert csa.attend_workspace_bytes(4) > 0
    assert csa.attend_workspace_bytes(4, window=129) == 0
    assert csa.attend_workspace_bytes(4, n_layers=9) == 0
    # pool: per candidate block of 4096 entries one count and 512 (block, fp64 max) records
    assert csa.hsi_pool_workspace_bytes(4, 1 << 20) >= 4 * 256 * 512 * 12
    assert csa.hsi_pool_workspace_bytes(0, 1 << 20) == 0
    # reindex: the MXFP4 variant's dequantised pool keys (16384 x 256 B per query) dominate
    assert csa.reindex_workspace_bytes(4) >= 4 * csa.HSI_POOL * 256
    assert csa.reindex_workspace_bytes(4, 256) == 0


# Fake, never-dereferenced, 16-byte-aligned addresses: every call below must be
# rejected by host validation, so nothing is launched and nothing is read.
P = ctypes.c_void_p(0x10000)
Q = ctypes.c_void_p(0x20000)
MIS = ctypes.c_void_p(0x10004)   # misaligned


def test_tile_max_stride(L):
    # ceil(N/16) tiles per row, padded to a multiple of 4 floats (16-byte rows)
    for N, ld in [(1, 4), (16, 4), (64, 4), (65, 8), (1000, 64), (1 << 20, 65536), (40001, 2504)]:
        assert L.csa2_tile_max_ld(N) == ld
        assert ld >= -(-N // 16) and ld % 4 == 0
    assert L.csa2_tile_max_ld(0) == 0


def _index(L, q=P, w=P, k=P, pos=None, ratio=1, T=4, qps=1, N=1024, s=P, tm=P, e=P, eb=1 << 20):
    return L.csa2_index(q, w, k, pos, ratio, T, qps, N, s, tm, e, eb, None)


def test_index_host_validation(L):
    assert _index(L, q=None) == INVALID
    assert _index(L, tm=None) == INVALID
    assert _index(L, s=MIS) == INVALID
    assert _index(L, e=None) == INVALID             # stats
    assert _index(L, e=MIS) == INVALID
    assert _index(L, k=MIS) == INVALID
    assert _index(L, T=0) == INVALID
    assert _index(L, T=4, qps=3) == INVALID
    assert _index(L, N=0) == INVALID
    assert _index(L, ratio=0) == INVALID
    assert _index(L, N=1 << 31) == UNSUPPORTED
    assert _index(L, eb=csa.index_stats_bytes(4, 1, 1024) - 1) == INVALID


# N large enough for the multi-pass regime, where a workspace is required, so
# that every call below is rejected by validation.
def _topk(L, s=None, tm=P, e=P, eb=1 << 30, q=P, w=P, k_idx=P, pos=None, ratio=1, T=4, qps=1, N=1 << 20, k=512,
          out=P, ws=P, wsb=None):
    if wsb is None:
        wsb = csa.topk_workspace_bytes(T, N, 512) or 1
    return L.csa2_topk(s, tm, e, eb, q, w, k_idx, pos, ratio, T, qps, N, k, out, ws, wsb, None)


def test_topk_host_validation(L):
    assert _topk(L, tm=None) == INVALID              # no scores and no tile maxima
    assert _topk(L, s=P, tm=None) == INVALID         # long rows always use the tile regime
    assert _topk(L, e=None) == INVALID              # stats
    assert _topk(L, eb=csa.index_stats_bytes(4, 1, 1 << 20) - 1) == INVALID
    assert _topk(L, tm=MIS) == INVALID
    assert _topk(L, out=MIS) == INVALID
    assert _topk(L, T=5, qps=2) == INVALID
    assert _topk(L, k=256) == UNSUPPORTED
    assert _topk(L, ws=None) == WORKSPACE
    assert _topk(L, wsb=csa.topk_min_workspace_bytes(4, 1 << 20) - 1) == WORKSPACE


def test_topk_select_mode_validation(L):
    def ex(select, ws=P, tm=P):
        wsb = csa.topk_workspace_bytes(4, 1 << 20, 512)
        return L.csa2_topk_ex(None, tm, P, 1 << 30, P, P, P, None, 1, 4, 1, 1 << 20, 512, select, P, ws, wsb, None)

    def ex_mx(select, ws=P):
        wsb = csa.topk_workspace_bytes(4, 1 << 20, 512)
        return L.csa2_topk_mxfp4_ex(None, P, P, 1 << 30, P, P, P, None, 1, 4, 1, 1 << 20, 512, select, P, ws, wsb,
                                    None)
    assert ex(2) == UNSUPPORTED and ex(-1) == UNSUPPORTED and ex_mx(2) == UNSUPPORTED
    # a valid mode reaches the usual checks (stopped here before any launch)
    assert ex(1, ws=None) == WORKSPACE and ex(0, ws=None) == WORKSPACE and ex_mx(1, ws=None) == WORKSPACE
    assert ex(1, tm=None) == INVALID


def _attend(L, q=P, kv=P, sc=P, idx=P, swa=P, end=P, sink=None, scale=0.044, T=4, qps=1, N=4096, S=128, W=128,
            k=512, out=P, lse=None, ws=P, wsb=1 << 30):
    return L.csa2_attend_fp4(q, kv, sc, idx, swa, end, sink, scale, T, qps, N, S, W, k, out, lse, ws, wsb, None)


def test_attend_host_validation(L):
    assert _attend(L, q=None) == INVALID
    assert _attend(L, swa=MIS) == INVALID
    assert _attend(L, scale=0.0) == INVALID
    assert _attend(L, scale=float("nan")) == INVALID
    assert _attend(L, scale=float("inf")) == INVALID
    assert _attend(L, S=0) == INVALID
    assert _attend(L, k=256) == UNSUPPORTED
    assert _attend(L, W=0) == UNSUPPORTED
    assert _attend(L, W=129) == UNSUPPORTED
    assert _attend(L, ws=None) == WORKSPACE
    assert _attend(L, wsb=csa.attend_workspace_bytes(4) - 1) == WORKSPACE


def test_reuse_host_validation(L):
    args = [P, P, P, P, P, P, None, 0.044, 4, 1, 4096, 128, 128, 512, P, None, P, 1 << 30, None]
    assert L.csa2_reuse_attend(0, *args) == UNSUPPORTED
    assert L.csa2_reuse_attend(9, *args) == UNSUPPORTED
    bad = list(args)
    bad[0] = None
    assert L.csa2_reuse_attend(2, *bad) == INVALID
    small = list(args)
    small[17] = csa.attend_workspace_bytes(4, n_layers=3) - 1
    assert L.csa2_reuse_attend(3, *small) == WORKSPACE


def _hsi(L, tm=P, e=P, eb=1 << 30, q=P, w=P, k_idx=P, pos=None, ratio=1, T=4, qps=1, N=1 << 20, out=P, ws=P,
         wsb=None):
    if wsb is None:
        wsb = csa.hsi_pool_workspace_bytes(T, N) or 1
    return L.csa2_hsi_pool(tm, e, eb, q, w, k_idx, pos, ratio, T, qps, N, out, ws, wsb, None)


def test_hsi_pool_host_validation(L):
    assert _hsi(L, tm=None) == INVALID
    assert _hsi(L, e=None) == INVALID
    assert _hsi(L, eb=csa.index_stats_bytes(4, 1, 1 << 20) - 1) == INVALID
    assert _hsi(L, out=MIS) == INVALID
    assert _hsi(L, T=5, qps=2) == INVALID
    assert _hsi(L, ratio=0) == INVALID
    assert _hsi(L, N=1 << 31) == UNSUPPORTED
    assert _hsi(L, ws=None) == WORKSPACE
    assert _hsi(L, wsb=csa.hsi_pool_workspace_bytes(4, 1 << 20) - 1) == WORKSPACE


def _reindex(L, pool=P, q=P, w=P, k_idx=P, T=4, qps=1, N=1 << 20, k=512, out=P, ws=P, wsb=None):
    if wsb is None:
        wsb = csa.reindex_workspace_bytes(T, 512) or 1
    return L.csa2_reindex(pool, q, w, k_idx, T, qps, N, k, out, ws, wsb, None)


def test_reindex_host_validation(L):
    assert _reindex(L, pool=None) == INVALID
    assert _reindex(L, pool=MIS) == INVALID
    assert _reindex(L, T=0) == INVALID
    assert _reindex(L, T=5, qps=2) == INVALID
    assert _reindex(L, k=256) == UNSUPPORTED
    assert _reindex(L, ws=None) == WORKSPACE
    assert _reindex(L, wsb=csa.reindex_workspace_bytes(4) - 1) == WORKSPACE


def test_mxfp4_host_validation(L):
    T, N = 4, 1 << 20
    sb = csa.index_mxfp4_stats_bytes(T, 1, N)
    # summary: header, at least 4096 group maxima per query, then the dequantised queries
    assert sb >= T * 16 + T * 4096 * 4 + T * 32 * 128 * 2
    assert csa.index_mxfp4_stats_bytes(4, 3, 100) == 0
    ix = lambda **kw: L.csa2_index_mxfp4(kw.get("qc", P), kw.get("qs", P), P, kw.get("kc", P), kw.get("ks", P), None,
                                         1, kw.get("T", T), 1, kw.get("N", N), None, P, P, kw.get("sb", sb), None)
    assert ix(qc=None) == INVALID
    assert ix(ks=MIS) == INVALID
    assert ix(T=0) == INVALID
    assert ix(N=1 << 31) == UNSUPPORTED
    assert ix(sb=sb - 1) == INVALID
    tk = lambda **kw: L.csa2_topk_mxfp4(None, kw.get("tm", P), P, kw.get("sb", sb), P, kw.get("kc", P), P, None, 1, T,
                                        1, N, kw.get("k", 512), P, kw.get("ws", P),
                                        kw.get("wsb", csa.topk_workspace_bytes(T, N)), None)
    assert tk(kc=None) == INVALID
    assert tk(tm=None) == INVALID
    assert tk(sb=sb - 1) == INVALID
    assert tk(k=256) == UNSUPPORTED
    assert tk(ws=None) == WORKSPACE
    hp = lambda **kw: L.csa2_hsi_pool_mxfp4(P, P, kw.get("sb", sb), P, P, P, None, 1, T, 1, N, P, kw.get("ws", P),
                                            csa.hsi_pool_workspace_bytes(T, N), None)
    assert hp(sb=sb - 1) == INVALID
    assert hp(ws=None) == WORKSPACE
    rx = lambda **kw: L.csa2_reindex_mxfp4(kw.get("pool", P), P, P, P, P, P, T, 1, N, kw.get("k", 512), P,
                                           kw.get("ws", P), csa.reindex_workspace_bytes(T), None)
    assert rx(pool=None) == INVALID
    assert rx(k=256) == UNSUPPORTED
    assert rx(ws=None) == WORKSPACE


def test_attend_ex_host_validation(L):
    O = csa._AttendOpts
    args = lambda opts, swa=P: [1, P, P, P, P, swa, P, None, 0.044, 4, 1, 4096, 128, 128, 512, opts, P, None, P,
                                1 << 30, None]
    assert L.csa2_attend_ex(*args(O(2, 0, None, None, None, None, 0.0))) == UNSUPPORTED     # unknown KV format
    assert L.csa2_attend_ex(*args(O(0, 2, None, None, None, None, 0.0))) == UNSUPPORTED     # unknown window format
    assert L.csa2_attend_ex(*args(O(0, 1, None, None, None, None, 0.0))) == INVALID         # FP8 window arrays missing
    assert L.csa2_attend_ex(*args(O(0, 1, 0x10004, 0x20000, 0x30000, None, 0.0), None)) == INVALID  # misaligned
    assert L.csa2_attend_ex(*args(O(0, 0, None, None, None, None, 0.0), None)) == INVALID   # bf16 window missing
    assert L.csa2_attend_ex(*args(O(0, 0, None, None, None, 0x40000, 1.0))) == INVALID      # rope base must be > 1
    assert L.csa2_attend_ex(*args(O(0, 0, None, None, None, 0x40000, float("inf")))) == INVALID
    bad = args(O(0, 0, None, None, None, None, 0.0))
    bad[0] = 9
    assert L.csa2_attend_ex(*bad) == UNSUPPORTED


def _kv_write(L, h=P, w_kv=P, w_z=P, w_ik=P, d=5120, n=4, m=2, pos=P, base=10000.0, kvf=0, codes=P,
              scales=P, kf=0, k_out=P, k_sc=None, ws=Q, wsb=None):
    if wsb is None:
        wsb = max(L.csa2_kv_write_workspace_bytes(n, m, d), 1)
    return L.csa2_kv_write(h, w_kv, w_z, w_ik, d, n, m, pos, base, kvf, codes, scales, kf, k_out, k_sc, ws, wsb,
                           None)


def test_kv_write_host_validation(L):
    # workspace: the slice sums of C (and Z for m > 1), fp32 per token and channel
    assert csa.kv_write_workspace_bytes(4, 1, 5120) >= 4 * 512 * 4
    assert csa.kv_write_workspace_bytes(300, 2, 5120) >= 2 * 600 * 512 * 4
    assert csa.kv_write_workspace_bytes(4, 3, 5120) == 0      # m in {1, 2, 4, 8}
    assert csa.kv_write_workspace_bytes(4, 1, 100) == 0       # d a multiple of 32
    assert csa.kv_write_workspace_bytes(0, 1, 512) == 0
    assert _kv_write(L, h=None) == INVALID
    assert _kv_write(L, w_z=None) == INVALID                  # gate weights needed for m > 1
    assert _kv_write(L, w_z=None, m=1, wsb=1) == WORKSPACE   # m = 1 takes no gate weights
    assert _kv_write(L, k_out=MIS) == INVALID
    assert _kv_write(L, kf=1) == INVALID                      # MXFP4 keys need their scale array
    assert _kv_write(L, base=1.0) == INVALID
    assert _kv_write(L, base=float("nan")) == INVALID
    assert _kv_write(L, n=0) == INVALID
    assert _kv_write(L, m=3) == UNSUPPORTED
    assert _kv_write(L, d=100) == UNSUPPORTED
    assert _kv_write(L, kvf=2) == UNSUPPORTED
    assert _kv_write(L, kf=2) == UNSUPPORTED
    assert _kv_write(L, ws=None) == WORKSPACE
    assert _kv_write(L, wsb=L.csa2_kv_write_workspace_bytes(4, 2, 5120) - 1) == WORKSPACE


def test_binding_fails_loudly_without_gpu_tensors():
    import torch
    with pytest.raises(ValueError):
        csa.csa2_index(torch.zeros(1, 32, 128, dtype=torch.bfloat16), torch.zeros(1, 32),
                       torch.zeros(1, 64, 128, dtype=torch.bfloat16))


def _attend_ex_cpu_args(T=2, N=64, S=130, fp8=True):
    """Host tensors shaped as csa2_attend_ex expects (one layer, MXFP4 main KV)."""
    import torch
    bf = torch.bfloat16
    a = dict(q=torch.zeros(T, csa.HEADS, csa.DIM, dtype=bf),
             kv_codes=torch.zeros(T, N, csa.DIM // 2, dtype=torch.uint8),
             kv_scales=torch.zeros(T, N, csa.DIM // 32, dtype=torch.uint8),
             indices=torch.zeros(T, csa.TOPK, dtype=torch.int32), swa_end=torch.zeros(T, dtype=torch.int32),
             rope_pos=torch.zeros(T, dtype=torch.int32))
    if fp8:
        a.update(swa_fp8=torch.zeros(T, S, 448, dtype=torch.uint8), swa_rope=torch.zeros(T, S, 64, dtype=bf),
                 swa_scales=torch.zeros(T, S, 8, dtype=torch.uint8))
    else:
        a.update(swa=torch.zeros(T, S, csa.DIM, dtype=bf))
    return a


@pytest.fixture
def host_binding(monkeypatch):
    """The binding with its device-type test and stream lookup taken out, so that its argument
    checks and marshalling can be exercised on host tensors (nothing is launched: calls are
    only recorded through bind())."""
    import torch
    seen = {}
    orig = csa._check

    def check(t, name, shape, elem_size=None, dtype=None, device=None):
        seen[name] = tuple(shape)
        if not isinstance(t, torch.Tensor):
            raise TypeError(name)
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if dtype is not None and t.dtype != dtype:
            raise TypeError(name)
        if elem_size is not None and t.element_size() != elem_size:
            raise TypeError(name)
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")

    monkeypatch.setattr(csa, "_check", check)
    monkeypatch.setattr(csa, "_stream", lambda t: None)
    assert orig is not check
    return seen


def test_attend_ex_checks_caller_outputs(host_binding):
    import torch
    a = _attend_ex_cpu_args()
    b = csa.bind(csa.csa2_attend_ex, **a, out=torch.zeros(2, csa.HEADS, csa.DIM, dtype=torch.bfloat16),
                 lse=torch.zeros(2, csa.HEADS))
    assert host_binding["out"] == (2, csa.HEADS, csa.DIM) and host_binding["lse"] == (2, csa.HEADS)
    assert isinstance(b.result, tuple)                      # a caller-supplied lse is returned
    with pytest.raises(ValueError):                          # short output buffer
        csa.bind(csa.csa2_attend_ex, **a, out=torch.zeros(1, csa.HEADS, csa.DIM, dtype=torch.bfloat16))
    with pytest.raises(TypeError):                           # wrong element size
        csa.bind(csa.csa2_attend_ex, **a, out=torch.zeros(2, csa.HEADS, csa.DIM))
    with pytest.raises(ValueError):                          # not contiguous
        o = torch.zeros(2, csa.DIM, csa.HEADS, dtype=torch.bfloat16).transpose(1, 2)
        csa.bind(csa.csa2_attend_ex, **a, out=o)
    with pytest.raises(ValueError):                          # lse of another layout
        csa.bind(csa.csa2_attend_ex, **a, lse=torch.zeros(2, csa.HEADS + 1))
    with pytest.raises(TypeError):
        csa.bind(csa.csa2_attend_ex, **a, lse=torch.zeros(2, csa.HEADS, dtype=torch.float64))


def test_attend_ex_window_must_be_given_once(host_binding):
    import torch
    a = _attend_ex_cpu_args()
    for k in ("swa_fp8", "swa_rope", "swa_scales"):
        a.pop(k)
    with pytest.raises(ValueError, match="window"):
        csa.bind(csa.csa2_attend_ex, **a)
    a["swa"] = torch.zeros(2, 130, csa.DIM, dtype=torch.bfloat16)
    a["swa_fp8"] = torch.zeros(2, 130, 448, dtype=torch.uint8)
    with pytest.raises(ValueError, match="window"):
        csa.bind(csa.csa2_attend_ex, **a)


def test_attend_ex_bind_keeps_option_tensors(host_binding):
    """The FP8 window arrays and the rotation positions travel in an options struct; bind()
    must hold them like every other tensor whose pointer it passes."""
    a = _attend_ex_cpu_args()
    b = csa.bind(csa.csa2_attend_ex, **a)
    held = {id(t) for t in b._tensors}
    for k in ("swa_fp8", "swa_rope", "swa_scales", "rope_pos", "q", "indices"):
        assert id(a[k]) in held, k
    (fn, args, name), = b._calls
    opts = args[15]._obj
    assert name == "csa2_attend_ex" and opts.swa_fp8 == a["swa_fp8"].data_ptr()
    assert opts.rope_pos == a["rope_pos"].data_ptr() and opts.swa_format == csa.SWA_FP8


@pytest.mark.skipif(os.environ.get("CSA2_SANITIZE", "") in ("", "0"), reason="sanitized CPU run not requested")
def test_sanitized_builds_are_loaded():
    """Under CSA2_SANITIZE=1 (with clang's ASan runtime preloaded) the suite runs the oracle and
    the library's host code built with AddressSanitizer and UndefinedBehaviorSanitizer."""
    import oracle
    csa.lib()
    oracle.lib()
    maps = open("/proc/self/maps").read()
    assert "libcsa2_san.so" in maps and "libcsa2_oracle_san.so" in maps
    assert "libclang_rt.asan" in maps


def test_static_attend_scratch_covers_every_call(L):
    """The split (and its partials) is chosen per launch shape and only used below 256
    query-layers: no valid call of csa2_reuse_attend_static needs more than its static scratch.
    Invalid layer counts are rejected before any device access (this host has no GPU)."""
    # one window per count of window chunks (the plan depends on the chunk count only)
    worst = max(csa.attend_workspace_bytes(T, window=w, n_layers=nl)
                for nl in range(1, 9) for w in (32, 64, 96, 128) for T in range(1, 300))
    assert 0 < worst <= 31_771_853 <= csa.STATIC_SCRATCH_BYTES        # 30.3 MiB, as documented
    assert all(csa.attend_workspace_bytes(T, n_layers=nl) == 0 for T in (256, 4096, 65535) for nl in (1, 8))
    assert csa.attend_workspace_bytes(128, n_layers=2) == 0             # 256 query-layers: not split
    # every split slot is one 64 x 512 bf16 partial plus its (max, sum) pair per head
    slot = 64 * 512 * 2 + 64 * 2 * 4
    for T, nl in [(4, 1), (4, 3), (32, 1), (32, 3), (64, 1), (160, 1)]:
        b = csa.attend_workspace_bytes(T, n_layers=nl)
        assert b % 256 == 0 and slot * T * nl * 2 <= b < slot * T * nl * 21   # 2 .. 20 items (chunks)
    P = ctypes.c_void_p(0x100000)
    args = lambda nl, T: [nl, P, P, P, P, P, P, None, 0.044, T, 1, 4096, 128, 128, 512, P, None, None]
    assert L.csa2_reuse_attend_static(*args(9, 4)) == UNSUPPORTED
    assert L.csa2_reuse_attend_static(*args(0, 4)) == UNSUPPORTED
