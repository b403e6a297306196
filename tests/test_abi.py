"""The C-ABI library loads, exports every entry point the header declares, and
rejects bad arguments on the host before anything reaches a GPU."""
import ctypes
import os
import re

import pytest

import sparse_attention_indexing_amd as lsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lsa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(lsa.LIB_PATH), reason="liblsa.so not built")

FAKE_DEV = ctypes.c_void_p(1 << 20)   # aligned address; init only records it


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\**\s+([a-z_0-9]+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert "build_bucket_cache" in names and "lsa_sparse_attention" in names
    assert len(names) >= 16
    L = ctypes.CDLL(lsa.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n


def _p(**kw):
    return lsa.Params(**kw)


def test_params_validation():
    L = lsa.lib()
    assert L.lsa_check_params(ctypes.byref(_p().c())) == 0
    for bad in [dict(d_latent=32), dict(n_pool=8), dict(block_keys=256), dict(n_buckets=32),
                dict(bucket_cap_keys=8), dict(k=-1), dict(k=9000), dict(window=0),
                dict(beam=513), dict(index_dtype=7), dict(start_level=-2), dict(mode=3), dict(exact_select=2)]:
        assert L.lsa_check_params(ctypes.byref(_p(**bad).c())) == -2, bad
    assert L.lsa_check_params(None) == -1
    d = lsa._Params()
    L.lsa_default_params(ctypes.byref(d))
    assert (d.d_latent, d.n_pool, d.block_keys, d.n_buckets, d.bucket_cap_keys) == (64, 4, 512, 64, 16)
    assert (d.k, d.n_sink, d.window) == (2048, 4, 512)


def test_sizes():
    assert lsa.list_len(_p(k=2048)) == 4 + 512 + 2048
    assert lsa.list_len(_p(k=4096)) == 4612
    assert lsa.top_buckets(_p(k=2048)) == 512 + 65
    assert lsa.top_buckets(_p(k=4096)) == 1089
    # the window's eligible blocks and the sinks' pooled items, worked by hand:
    # window 2,048 reaches back into ceil(2,047 / 512) = 4 eligible blocks
    assert lsa.top_buckets(_p(k=256, window=2048)) == 64 + 4 * 64 + 1
    assert lsa.top_buckets(_p(k=2048, n_sink=64)) == 512 + 64 + 16
    assert lsa.top_buckets(_p(k=2048, n_sink=0, window=1)) == 512        # only the query itself
    assert lsa.top_buckets(_p(k=2048, n_sink=5, window=513)) == 512 + 64 + 2
    assert lsa.top_buckets(_p(k=2048, window=514)) == 512 + 128 + 1
    # every candidate of a query must fit one workgroup (9 cap + 4 k bytes of LDS)
    assert lsa.top_buckets(_p(k=8192, window=4096)) == 2048 + 512 + 1
    assert lsa.top_buckets(_p(k=8192, window=8192)) == 2048 + 1024 + 1      # cap 10,240
    # the scans: ceil(k / b) + ceil(n_sink / b) runs
    assert lsa.top_buckets(_p(k=4096, scan_keys=1)) == 4100                  # cap 13,312
    assert lsa.top_buckets(_p(k=2048, scan_keys=8)) == 256 + 1
    assert lsa.top_buckets(_p(k=2048, scan_keys=4, n_sink=5)) == 512 + 2
    for bad in [dict(scan_keys=2), dict(scan_keys=1, mode=1), dict(scan_keys=4, window=511),
                dict(scan_keys=1, k=8192), dict(score_heads=3), dict(score_heads=16),
                dict(score_heads=8, mode=1), dict(score_heads=8, index_dtype=0),
                dict(score_heads=2, scan_keys=4)]:
        assert lsa.lib().lsa_check_params(ctypes.byref(_p(**bad).c())) == -2, bad
    from oracle import lsa_oracle as O
    for k in (0, 1, 255, 2048, 4096):
        for window in (1, 2, 511, 512, 513, 1024, 2048):
            for n_sink in (0, 1, 4, 5, 64):
                assert lsa.top_buckets(_p(k=k, window=window, n_sink=n_sink)) == O.Params(
                    k=k, window=window, n_sink=n_sink).top_b, (k, window, n_sink)
    L = lsa.lib()
    for bad in [dict(k=8192, n_sink=8192), dict(k=8192, window=8192, n_sink=8192)]:
        assert L.lsa_check_params(ctypes.byref(_p(**bad).c())) == -2, bad
    L = lsa.lib()
    flat = L.lsa_cache_bytes(ctypes.byref(_p().c()), 1 << 20)
    tree = L.lsa_cache_bytes(ctypes.byref(_p(mode=lsa.LSA_TREE).c()), 1 << 20)
    nb = (1 << 20) // 512 * 64
    assert flat >= nb * (128 + 4)
    assert tree > flat + (nb - 1) * 128
    # bf16 centroids + 4-byte member tables: 16.5 bytes per token
    assert flat / (1 << 20) < 17.0
    assert L.lsa_cache_bytes(ctypes.byref(_p().c()), -1) == -1
    assert L.lsa_index_workspace_bytes(ctypes.byref(_p().c()), 100) > 100 * 2048 * 8


def test_cache_init_and_host_errors():
    L = lsa.lib()
    p = _p()
    need = L.lsa_cache_bytes(ctypes.byref(p.c()), 4096)
    h = ctypes.c_void_p()
    assert L.lsa_cache_init(ctypes.byref(p.c()), 4096, FAKE_DEV, need - 1, ctypes.byref(h)) == -4
    assert L.lsa_cache_init(ctypes.byref(p.c()), 4096, None, need, ctypes.byref(h)) == -1
    assert L.lsa_cache_init(ctypes.byref(p.c()), 4096, ctypes.c_void_p((1 << 20) + 8), need,
                            ctypes.byref(h)) == -1
    assert L.lsa_cache_init(ctypes.byref(p.c()), 4096, FAKE_DEV, need, ctypes.byref(h)) == 0
    try:
        assert L.lsa_cache_tokens(h) == 0
        # nothing to do / over capacity / null keys: all decided on the host
        assert L.build_bucket_cache(h, None, 0, None) == 0
        assert L.build_bucket_cache(h, FAKE_DEV, 5000, None) == -4
        assert L.build_bucket_cache(h, None, 10, None) == -1
        assert L.build_bucket_cache(h, FAKE_DEV, -1, None) == -1
        ws = L.lsa_index_workspace_bytes(ctypes.byref(p.c()), 8)
        # queries past the clustered blocks
        assert L.lsa_index_prefill(h, FAKE_DEV, 1000, 8, ctypes.byref(p.c()), FAKE_DEV, FAKE_DEV,
                                   None, FAKE_DEV, ws, None) == -6
        # workspace too small
        assert L.lsa_index_prefill(h, FAKE_DEV, 0, 8, ctypes.byref(p.c()), FAKE_DEV, FAKE_DEV,
                                   None, FAKE_DEV, ws - 1, None) == -3
        # tree query on a flat cache; dtype mismatch
        assert L.lsa_index_prefill(h, FAKE_DEV, 0, 8, ctypes.byref(_p(mode=1).c()), FAKE_DEV,
                                   FAKE_DEV, None, FAKE_DEV, ws, None) == -6
        assert L.lsa_index_prefill(h, FAKE_DEV, 0, 8, ctypes.byref(_p(index_dtype=0).c()),
                                   FAKE_DEV, FAKE_DEV, None, FAKE_DEV, 1 << 30, None) == -1
        arr = (ctypes.c_void_p * 2)(h, h)
        assert L.lsa_index_decode(arr, 2, FAKE_DEV, FAKE_DEV, ctypes.byref(p.c()), FAKE_DEV,
                                  FAKE_DEV, FAKE_DEV, 1 << 30, None) == -1   # same cache twice
        assert L.lsa_index_decode(arr, 65, FAKE_DEV, FAKE_DEV, ctypes.byref(p.c()), FAKE_DEV,
                                  FAKE_DEV, FAKE_DEV, 1 << 30, None) == -1
        assert L.lsa_cache_tokens(h) == 0     # rejected calls changed nothing
    finally:
        assert L.lsa_cache_release(h) == 0


def test_attention_host_errors():
    L = lsa.lib()
    f = ctypes.c_float(0.1)
    args = lambda D=128, Hq=32, Hkv=4, dt=1, splits=1, ws=0: (
        FAKE_DEV, FAKE_DEV, FAKE_DEV, 1, 16, 1024, Hq, Hkv, D, FAKE_DEV, FAKE_DEV, 100, f, dt,
        splits, FAKE_DEV, None, ws, None)
    assert L.lsa_sparse_attention(*args(D=64)) == -2
    assert L.lsa_sparse_attention(*args(Hq=30)) == -2
    assert L.lsa_sparse_attention(*args(Hq=64, Hkv=2)) == -2
    assert L.lsa_sparse_attention(*args(dt=5)) == -2
    assert L.lsa_sparse_attention(*args(splits=0)) == -1
    assert L.lsa_sparse_attention(*args(splits=4)) == -3
    empty_cache = list(args())
    empty_cache[5] = 0                     # Tmax = 0 with rows to attend
    assert L.lsa_sparse_attention(*empty_cache) == -1
    assert lsa.attention_launch_rows() == 1024
    # per-(row, KV head) workgroups for bf16, 4 KV heads, caches of <= 256 MiB each
    hm = lambda B, T, Hkv=4, D=128, dt=lsa.LSA_BF16: lsa.attention_head_major(B, T, Hkv, D, dt)
    assert hm(1, 131072) and hm(1, 262144) and not hm(1, 262145)
    assert hm(2, 131072) and not hm(2, 131073) and hm(0, 10**9) and hm(7, 0)
    assert not hm(1, 1 << 20) and not hm(16, 1 << 20) and not hm(1, 10**7)
    assert not hm(1, 4096, dt=lsa.LSA_F32) and not hm(1, 4096, D=64) and not hm(1, 4096, Hkv=0)
    assert hm(1, 4096, Hkv=8) and hm(16, 1 << 20, Hkv=1) and hm(1, 10**7, Hkv=3)
    assert not hm(1 << 30, 1 << 32) and not hm(-1, 4) and not hm(1, -4)
    assert L.lsa_attention_workspace_bytes(1, 16, 32, 128, 1) == 0
    assert L.lsa_attention_workspace_bytes(1, 16, 32, 128, 4) == 16 * 4 * 32 * 130 * 4
    assert L.lsa_status_string(-3) == b"workspace too small"


def test_static_attention_host_errors():
    """The allocation-free attention checks its arguments like the other entry
    point and rejects split partials beyond its fixed array, all on the host
    before anything is launched."""
    L = lsa.lib()
    f = ctypes.c_float(0.1)
    args = lambda D=128, Hq=32, Hkv=4, dt=1, splits=1, rows=16: (
        FAKE_DEV, FAKE_DEV, FAKE_DEV, 1, rows, 1024, Hq, Hkv, D, FAKE_DEV, FAKE_DEV, 100, f, dt,
        splits, FAKE_DEV, None)
    assert L.lsa_sparse_attention_static(*args(D=64)) == -2
    assert L.lsa_sparse_attention_static(*args(Hq=30)) == -2
    assert L.lsa_sparse_attention_static(*args(dt=5)) == -2
    assert L.lsa_sparse_attention_static(*args(splits=0)) == -1
    assert L.lsa_sparse_attention_static(*args(rows=0)) == 0          # nothing to do
    # partials of 64 rows x 64 splits x 32 heads x 130 floats = 68 MB > 16 MiB
    assert L.lsa_attention_workspace_bytes(1, 64, 32, 128, 64) > (16 << 20)
    assert L.lsa_sparse_attention_static(*args(rows=64, splits=64)) == -4
    assert L.lsa_sparse_attention_static(FAKE_DEV, FAKE_DEV, FAKE_DEV, 1, 16, 1024, 32, 4, 128,
                                         None, FAKE_DEV, 100, f, 1, 1, FAKE_DEV, None) == -1


def test_dense_attention_host_errors():
    L = lsa.lib()
    f = ctypes.c_float(0.1)
    args = lambda Tq=16, q_start=0, Tk=1024, Hq=32, Hkv=4, D=128, band=1 << 40, dt=1: (
        FAKE_DEV, FAKE_DEV, FAKE_DEV, Tq, q_start, Tk, Hq, Hkv, D, band, f, dt, FAKE_DEV, None)
    assert L.lsa_dense_attention(*args(D=64)) == -2
    assert L.lsa_dense_attention(*args(Hq=24, Hkv=1)) == -2      # group of 24
    assert L.lsa_dense_attention(*args(dt=0)) == -2
    assert L.lsa_dense_attention(*args(band=0)) == -1
    assert L.lsa_dense_attention(*args(q_start=1020)) == -1      # rows past the keys
    assert L.lsa_dense_attention(*args(Tq=0)) == 0


def test_prefill_attention_host_errors():
    """lsa_sparse_attention_prefill rejects fp32, other group sizes, rows past
    the cache, bad sink/window counts and a short workspace on the host,
    before anything is launched."""
    L = lsa.lib()
    f = ctypes.c_float(0.1)
    need = L.lsa_prefill_attention_workspace_bytes(1, 16, 32, 128)
    assert need == 16 * 32 * 130 * 4
    # the near state of one group of four launches at most: 4,096 rows
    assert L.lsa_prefill_attention_workspace_bytes(2, 100000, 32, 128) == 4096 * 32 * 130 * 4
    assert L.lsa_prefill_attention_workspace_bytes(1, 16, 32, 64) == -1
    args = lambda Tq=16, q_start=0, Tmax=1024, Hq=32, Hkv=4, D=128, n_sink=4, window=512, dt=1, \
        ws=need: (FAKE_DEV, FAKE_DEV, FAKE_DEV, 1, Tq, q_start, Tmax, Hq, Hkv, D, FAKE_DEV, FAKE_DEV,
                  100, n_sink, window, f, dt, FAKE_DEV, FAKE_DEV, ws, None)
    assert L.lsa_sparse_attention_prefill(*args(dt=0)) == -2
    assert L.lsa_sparse_attention_prefill(*args(D=64)) == -2
    assert L.lsa_sparse_attention_prefill(*args(Hq=12, Hkv=4)) == -2     # group of 3
    assert L.lsa_sparse_attention_prefill(*args(q_start=1010)) == -1     # rows past the cache
    assert L.lsa_sparse_attention_prefill(*args(window=0)) == -1
    assert L.lsa_sparse_attention_prefill(*args(n_sink=-1)) == -1
    assert L.lsa_sparse_attention_prefill(*args(ws=need - 1)) == -3
    assert L.lsa_sparse_attention_prefill(*args(Tq=0)) == 0
