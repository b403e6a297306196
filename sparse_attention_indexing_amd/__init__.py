"""Python binding of the LSA C ABI (include/lsa.h), one function per entry point.

Argument marshalling only: every step of the path runs in the HIP library
``liblsa.so`` built in-tree for gfx950.  PyTorch tensors provide device
memory and the current HIP stream.  There is no fallback: if the library is
missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, fields

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liblsa.so")

LSA_F32, LSA_BF16 = 0, 1
LSA_FLAT, LSA_TREE = 0, 1
_STATUS = {0: "ok", -1: "invalid argument", -2: "unsupported", -3: "workspace too small",
           -4: "capacity exceeded", -5: "HIP error", -6: "bad cache state"}


class LsaError(RuntimeError):
    def __init__(self, fn, code):
        super().__init__(f"{fn} failed: {code} ({_STATUS.get(code, 'unknown')})")
        self.code = code


class _Params(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "d_latent", "n_pool", "block_keys", "n_buckets", "bucket_cap_keys", "k", "n_sink",
        "window", "mode", "beam", "leaf_level", "index_dtype", "exact_select", "scan_keys",
        "score_heads", "start_level")]


class _View(ctypes.Structure):
    _fields_ = [("n_tokens", ctypes.c_int64), ("n_blocks", ctypes.c_int64),
                ("n_buckets", ctypes.c_int64), ("centroids", ctypes.c_void_p),
                ("members", ctypes.c_void_p), ("staging", ctypes.c_void_p),
                ("tree_height", ctypes.c_int32), ("level_nodes", ctypes.c_int64 * 32),
                ("level_centroids", ctypes.c_void_p * 32), ("level_child", ctypes.c_void_p * 32),
                ("level_min_block", ctypes.c_void_p * 32)]


@dataclass
class Params:
    """Method parameters (see lsa_params in include/lsa.h)."""
    k: int = 2048
    n_sink: int = 4
    window: int = 512
    mode: int = LSA_FLAT
    beam: int = 64
    leaf_level: int = -1
    index_dtype: int = LSA_BF16
    exact_select: int = 0
    scan_keys: int = 0            # 0: LSA buckets; 1 / 4 / 8: token / block scan baseline
    score_heads: int = 0          # 2 / 4 / 8: query heads per position, max-over-heads scores
    start_level: int = -1         # tree: level scored in full first (-1: start at the root)
    d_latent: int = 64
    n_pool: int = 4
    block_keys: int = 512
    n_buckets: int = 64
    bucket_cap_keys: int = 16

    def c(self) -> _Params:
        return _Params(**{f.name: int(getattr(self, f.name)) for f in fields(self)})


_lib = None


def lib():
    """The loaded liblsa.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} not found: build it with "
                           "`python -m sparse_attention_indexing_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, i64, i32, vp = ctypes.POINTER(_Params), ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
    sig = {
        "lsa_default_params": (None, [P]),
        "lsa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "lsa_check_params": (ctypes.c_int, [P]),
        "lsa_list_len": (i32, [P]),
        "lsa_top_buckets": (i32, [P]),
        "lsa_cache_bytes": (i64, [P, i64]),
        "lsa_cache_init": (ctypes.c_int, [P, i64, vp, i64, ctypes.POINTER(vp)]),
        "lsa_cache_release": (ctypes.c_int, [vp]),
        "lsa_cache_tokens": (i64, [vp]),
        "lsa_cache_get_view": (ctypes.c_int, [vp, ctypes.POINTER(_View)]),
        "build_bucket_cache": (ctypes.c_int, [vp, vp, i64, vp]),
        "lsa_index_workspace_bytes": (i64, [P, i64]),
        "lsa_index_status_offset": (i64, [P, i64]),
        "lsa_index_prefill": (ctypes.c_int, [vp, vp, i64, i64, P, vp, vp, vp, vp, i64, vp]),
        "lsa_index_decode": (ctypes.c_int, [ctypes.POINTER(vp), i32, vp, vp, P, vp, vp, vp, i64, vp]),
        "lsa_attention_workspace_bytes": (i64, [i32, i64, i32, i32, i32]),
        "lsa_attention_default_splits": (i32, [i64, i32]),
        "lsa_sparse_attention": (ctypes.c_int, [vp, vp, vp, i32, i64, i64, i32, i32, i32, vp, vp,
                                                i32, ctypes.c_float, i32, i32, vp, vp, i64, vp]),
        "lsa_sparse_attention_static": (ctypes.c_int, [vp, vp, vp, i32, i64, i64, i32, i32, i32, vp,
                                                       vp, i32, ctypes.c_float, i32, i32, vp, vp]),
        "lsa_dense_attention": (ctypes.c_int, [vp, vp, vp, i64, i64, i64, i32, i32, i32, i64,
                                               ctypes.c_float, i32, vp, vp]),
        "lsa_prefill_attention_workspace_bytes": (i64, [i32, i64, i32, i32]),
        "lsa_sparse_attention_prefill": (ctypes.c_int, [vp, vp, vp, i32, i64, i64, i64, i32, i32,
                                                        i32, vp, vp, i32, i32, i32, ctypes.c_float,
                                                        i32, vp, vp, i64, vp]),
        "lsa_attention_launch_rows": (i64, []),
        "lsa_attention_head_major": (i32, [i32, i64, i32, i32, i32]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    L.lsa_params_bytes.restype = i32
    L.lsa_params_bytes.argtypes = []
    if L.lsa_params_bytes() != ctypes.sizeof(_Params):
        raise RuntimeError(f"{LIB_PATH} was built with another lsa_params layout "
                           f"({L.lsa_params_bytes()} bytes, the binding has "
                           f"{ctypes.sizeof(_Params)}): rebuild the library")
    _lib = L
    return L


def _check(fn, rc):
    if rc < 0:
        raise LsaError(fn, int(rc))
    return rc


def _stream(device=None) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, dtype, name):
    if not t.is_cuda or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous CUDA {dtype} tensor")


def list_len(p: Params) -> int:
    return _check("lsa_list_len", lib().lsa_list_len(ctypes.byref(p.c())))


def attention_default_splits(rows: int, L_max: int) -> int:
    return int(lib().lsa_attention_default_splits(rows, L_max))


def top_buckets(p: Params) -> int:
    return _check("lsa_top_buckets", lib().lsa_top_buckets(ctypes.byref(p.c())))


def index_workspace_bytes(p: Params, n: int) -> int:
    return _check("lsa_index_workspace_bytes", lib().lsa_index_workspace_bytes(ctypes.byref(p.c()), n))


def exact_fallbacks(p: Params, n: int, workspace: torch.Tensor) -> int:
    """How many of the n queries of the last index call on `workspace` had their
    bucket selection redone exactly (lsa_index_status_offset).  Synchronises."""
    off = _check("lsa_index_status_offset", lib().lsa_index_status_offset(ctypes.byref(p.c()), n))
    return int(workspace[off:off + 4 * n].view(torch.int32).sum().item())


class BucketCache:
    """A bucket cache in caller-owned device memory (a torch uint8 tensor)."""

    def __init__(self, p: Params, max_tokens: int, device="cuda"):
        self.params = p
        nbytes = _check("lsa_cache_bytes", lib().lsa_cache_bytes(ctypes.byref(p.c()), max_tokens))
        self.mem = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
        h = ctypes.c_void_p()
        _check("lsa_cache_init", lib().lsa_cache_init(ctypes.byref(p.c()), max_tokens, _ptr(self.mem),
                                                       nbytes, ctypes.byref(h)))
        self.handle = h

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and _lib is not None:
            _lib.lsa_cache_release(h)
            self.handle = None

    @property
    def n_tokens(self) -> int:
        return _check("lsa_cache_tokens", lib().lsa_cache_tokens(self.handle))

    def build(self, latent_keys: torch.Tensor) -> None:
        """build_bucket_cache: append keys [n, 64] fp32 and cluster full blocks."""
        _need(latent_keys, torch.float32, "latent_keys")
        _check("build_bucket_cache", lib().build_bucket_cache(
            self.handle, _ptr(latent_keys), latent_keys.shape[0], ctypes.c_void_p(_stream())))

    def view(self) -> dict:
        """Device tensors aliasing the cache contents (for reading it back)."""
        v = _View()
        _check("lsa_cache_get_view", lib().lsa_cache_get_view(self.handle, ctypes.byref(v)))
        base = self.mem.data_ptr()
        bf16 = self.params.index_dtype == LSA_BF16
        esz = 2 if bf16 else 4
        dt = torch.bfloat16 if bf16 else torch.float32

        def sub(addr, nbytes, dtype, shape):
            off = addr - base
            return self.mem[off:off + nbytes].view(dtype).view(*shape)

        nb = v.n_buckets
        out = dict(n_tokens=v.n_tokens, n_blocks=v.n_blocks, n_buckets=nb,
                   centroids=sub(v.centroids, nb * 64 * esz, dt, (nb, 64)),
                   members=None if not v.members else sub(v.members, nb * 4, torch.int32, (nb,)),
                   tree_height=v.tree_height, levels=[])
        for l in range(1, v.tree_height + 1):
            n = v.level_nodes[l]
            out["levels"].append(dict(
                centroids=sub(v.level_centroids[l], n * 64 * esz, dt, (n, 64)),
                child=sub(v.level_child[l], n * 8, torch.int32, (n, 2)),
                min_block=sub(v.level_min_block[l], n * 4, torch.int32, (n,))))
        return out


def index_prefill(cache: BucketCache, latent_q: torch.Tensor, q_start: int, p: Params,
                  ranked: bool = False, workspace: torch.Tensor | None = None,
                  out: tuple | None = None, stats: dict | None = None):
    """lsa_index_prefill -> (idx [Tq, L] int32, count [Tq] int32[, ranked [Tq, B]]).
    With `stats`, stats["exact_fallbacks"] receives the number of queries whose
    bucket selection took the exact fallback (this synchronises)."""
    _need(latent_q, torch.float32, "latent_q")
    Tq = latent_q.shape[0]
    if p.score_heads > 1 and (latent_q.dim() != 3 or latent_q.shape[1] != p.score_heads):
        raise ValueError("latent_q must be [Tq, score_heads, 64] with several query heads")
    L = list_len(p)
    dev = latent_q.device
    if out is None:
        idx = torch.empty((Tq, L), dtype=torch.int32, device=dev)
        cnt = torch.empty((Tq,), dtype=torch.int32, device=dev)
    else:
        idx, cnt = out
    rk = torch.empty((Tq, top_buckets(p)), dtype=torch.int32, device=dev) if ranked else None
    wsb = index_workspace_bytes(p, Tq)
    if workspace is None or workspace.numel() < wsb:
        workspace = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    _check("lsa_index_prefill", lib().lsa_index_prefill(
        cache.handle, _ptr(latent_q), q_start, Tq, ctypes.byref(p.c()), _ptr(idx), _ptr(cnt),
        _ptr(rk), _ptr(workspace), workspace.numel(), ctypes.c_void_p(_stream())))
    if stats is not None:
        stats["exact_fallbacks"] = exact_fallbacks(p, Tq, workspace)
    return (idx, cnt, rk) if ranked else (idx, cnt)


def index_decode(caches: list, latent_q: torch.Tensor, latent_k_new: torch.Tensor, p: Params,
                 workspace: torch.Tensor | None = None, out: tuple | None = None,
                 stats: dict | None = None):
    """lsa_index_decode -> (idx [B, L] int32, count [B] int32).  With `stats`,
    stats["exact_fallbacks"] receives the number of sequences whose bucket
    selection took the exact fallback (this synchronises)."""
    _need(latent_q, torch.float32, "latent_q")
    _need(latent_k_new, torch.float32, "latent_k_new")
    B = len(caches)
    L = list_len(p)
    dev = latent_q.device
    if out is None:
        idx = torch.empty((B, L), dtype=torch.int32, device=dev)
        cnt = torch.empty((B,), dtype=torch.int32, device=dev)
    else:
        idx, cnt = out
    wsb = index_workspace_bytes(p, B)
    if workspace is None or workspace.numel() < wsb:
        workspace = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    arr = (ctypes.c_void_p * B)(*[c.handle for c in caches])
    _check("lsa_index_decode", lib().lsa_index_decode(
        arr, B, _ptr(latent_q), _ptr(latent_k_new), ctypes.byref(p.c()), _ptr(idx), _ptr(cnt),
        _ptr(workspace), workspace.numel(), ctypes.c_void_p(_stream())))
    if stats is not None:
        stats["exact_fallbacks"] = exact_fallbacks(p, B, workspace)
    return idx, cnt


def sparse_attention(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                     idx: torch.Tensor, count: torch.Tensor, scale: float | None = None,
                     splits: int = 1, out: torch.Tensor | None = None,
                     workspace: torch.Tensor | None = None) -> torch.Tensor:
    """lsa_sparse_attention.  q [B, Tq, Hq, D], k/v [B, Tmax, Hkv, D] (3-d inputs
    mean B = 1), idx [B, Tq, L] / [Tq, L], count [B, Tq] / [Tq]."""
    squeeze = q.dim() == 3
    if squeeze:
        q, k_cache, v_cache = q[None], k_cache[None], v_cache[None]
    B, Tq, Hq, D = q.shape
    _, Tmax, Hkv, _ = k_cache.shape
    if q.dtype == torch.bfloat16:
        dt = LSA_BF16
    elif q.dtype == torch.float32:
        dt = LSA_F32
    else:
        raise ValueError("q must be bf16 or fp32")
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, q.dtype, n)
    _need(idx, torch.int32, "idx")
    _need(count, torch.int32, "count")
    L = idx.shape[-1]
    if out is None:
        out = torch.empty_like(q)
    scale = 1.0 / D ** 0.5 if scale is None else scale
    wsb = _check("lsa_attention_workspace_bytes",
                 lib().lsa_attention_workspace_bytes(B, Tq, Hq, D, splits))
    if wsb > 0 and (workspace is None or workspace.numel() < wsb):
        workspace = torch.empty(wsb, dtype=torch.uint8, device=q.device)
    _check("lsa_sparse_attention", lib().lsa_sparse_attention(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), B, Tq, Tmax, Hq, Hkv, D, _ptr(idx), _ptr(count),
        L, ctypes.c_float(scale), dt, splits, _ptr(out), _ptr(workspace) if wsb > 0 else None,
        workspace.numel() if wsb > 0 else 0, ctypes.c_void_p(_stream())))
    return out[0] if squeeze else out


def sparse_attention_prefill(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                             idx: torch.Tensor, count: torch.Tensor, q_start: int, p: "Params",
                             scale: float | None = None, out: torch.Tensor | None = None,
                             workspace: torch.Tensor | None = None) -> torch.Tensor:
    """lsa_sparse_attention_prefill: attention of a prefill chunk (positions
    q_start ..) over each row's near set (p.n_sink sinks, p.window window) and
    its list's other entries.  bf16; shapes as for sparse_attention."""
    squeeze = q.dim() == 3
    if squeeze:
        q, k_cache, v_cache = q[None], k_cache[None], v_cache[None]
    B, Tq, Hq, D = q.shape
    _, Tmax, Hkv, _ = k_cache.shape
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, torch.bfloat16, n)
    _need(idx, torch.int32, "idx")
    _need(count, torch.int32, "count")
    L = idx.shape[-1]
    if out is None:
        out = torch.empty_like(q)
    scale = 1.0 / D ** 0.5 if scale is None else scale
    wsb = _check("lsa_prefill_attention_workspace_bytes",
                 lib().lsa_prefill_attention_workspace_bytes(B, Tq, Hq, D))
    if workspace is None or workspace.numel() < wsb:
        workspace = torch.empty(max(wsb, 1), dtype=torch.uint8, device=q.device)
    _check("lsa_sparse_attention_prefill", lib().lsa_sparse_attention_prefill(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), B, Tq, q_start, Tmax, Hq, Hkv, D, _ptr(idx),
        _ptr(count), L, p.n_sink, p.window, ctypes.c_float(scale), LSA_BF16, _ptr(out),
        _ptr(workspace), workspace.numel(), ctypes.c_void_p(_stream())))
    return out[0] if squeeze else out


def sparse_attention_static(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                            idx: torch.Tensor, count: torch.Tensor, scale: float | None = None,
                            splits: int = 1, out: torch.Tensor | None = None) -> torch.Tensor:
    """lsa_sparse_attention_static: lsa_sparse_attention with the split partials
    in the library's fixed device array (no workspace; allocates nothing when
    `out` is given).  Shapes as for sparse_attention."""
    squeeze = q.dim() == 3
    if squeeze:
        q, k_cache, v_cache = q[None], k_cache[None], v_cache[None]
    B, Tq, Hq, D = q.shape
    _, Tmax, Hkv, _ = k_cache.shape
    if q.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("q must be bf16 or fp32")
    dt = LSA_BF16 if q.dtype == torch.bfloat16 else LSA_F32
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, q.dtype, n)
    _need(idx, torch.int32, "idx")
    _need(count, torch.int32, "count")
    if out is None:
        out = torch.empty_like(q)
    elif squeeze:
        out = out[None]
    scale = 1.0 / D ** 0.5 if scale is None else scale
    _check("lsa_sparse_attention_static", lib().lsa_sparse_attention_static(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), B, Tq, Tmax, Hq, Hkv, D, _ptr(idx), _ptr(count),
        idx.shape[-1], ctypes.c_float(scale), dt, splits, _ptr(out), ctypes.c_void_p(_stream())))
    return out[0] if squeeze else out


def dense_attention(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, q_start: int,
                    band: int | None = None, scale: float | None = None,
                    out: torch.Tensor | None = None) -> torch.Tensor:
    """lsa_dense_attention: q [Tq, Hq, 128] at positions q_start.., k/v [Tk, Hkv, 128]
    (bf16); every query attends to keys [max(0, p - band + 1), p] (band None:
    every earlier key)."""
    Tq, Hq, D = q.shape
    Tk, Hkv, _ = k_cache.shape
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, torch.bfloat16, n)
    if out is None:
        out = torch.empty_like(q)
    scale = 1.0 / D ** 0.5 if scale is None else scale
    band = (1 << 62) if band is None else band
    _check("lsa_dense_attention", lib().lsa_dense_attention(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), Tq, q_start, Tk, Hq, Hkv, D, band,
        ctypes.c_float(scale), LSA_BF16, _ptr(out), ctypes.c_void_p(_stream())))
    return out


def attention_launch_rows() -> int:
    """lsa_attention_launch_rows: query rows per bf16 attention launch."""
    return int(lib().lsa_attention_launch_rows())


def attention_head_major(B: int, Tmax: int, Hkv: int, D: int, dtype: int) -> bool:
    """lsa_attention_head_major: whether attention over these shapes runs one
    workgroup per (query row, KV head)."""
    return bool(lib().lsa_attention_head_major(B, Tmax, Hkv, D, dtype))


__all__ = ["Params", "BucketCache", "index_prefill", "index_decode", "sparse_attention",
           "sparse_attention_static", "dense_attention",
           "attention_launch_rows", "attention_head_major",
           "list_len", "top_buckets", "index_workspace_bytes", "exact_fallbacks", "lib",
           "LsaError",
           "LSA_F32", "LSA_BF16", "LSA_FLAT", "LSA_TREE"]
