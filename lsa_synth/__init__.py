"""Seeded synthetic inputs for the LSA indexing + sparse-attention path.

This module only *draws* inputs.  It holds none of the method's arithmetic
(no normalisation of keys, no clustering, no scoring, no attention), so the
CPU oracle and the HIP library can both be fed from it without sharing any
code with each other.

Workloads (one attention layer each):

  cfg 1  T=4,096 fp32 parity case: 64-component latent mixture, 4 query heads,
         1 KV head, head_dim 128, flat search, k=256.
  cfg 2  T=131,072 prefill, bf16 K/V, 32 query / 4 KV heads, 1,024 components,
         flat search, k=2,048.
  cfg 3  decode: 16 independent sequences with T=1,048,576 cached tokens each,
         4,096 components, k=2,048, flat search.
  cfg 4  T=1,048,576 context, last 8,192 queries, tree search (beam 64) and flat
         search on the same inputs, 1,024 components, k=2,048.
  cfg 5  T=10,000,000 context, last 32,768 queries (and batch-1 decode), 16,384
         components, k=4,096, flat and tree.

Latent index keys / queries (64-d): a mixture of isotropic Gaussians around
unit-norm means, sigma 0.3 per coordinate, with each token's component drawn
in runs of 1..32 consecutive tokens (most buckets on real text are runs of
neighbouring tokens; 72x post, "Latent Sparse Attention: 72x in One Layer..."
introduction and "What our test showed").

Q/K/V entries are N(0,1), drawn with the counter-based Philox4x32-10
generator (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as
1, 2, 3", SC 2011) followed by the Box-Muller transform in fp64, then rounded
to nearest-even in the storage dtype.  Every element is a pure function of
(key, element index), so the host can draw any subset of rows the oracle
needs and the device can draw the full tensors (see ``device_fill_normal``).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field

import numpy as np

SEED = 20261030
_ROW_CHUNK = 65536  # latent rows per independently seeded chunk


@dataclass(frozen=True)
class Workload:
    cfg: int
    name: str
    T: int                 # context length (cached tokens for decode)
    n_comp: int            # mixture components of the latent keys/queries
    Hq: int
    Hkv: int
    D: int
    k: int                 # far keys per query
    dtype: str             # "f32" | "bf16": K/V/Q storage and index dtype
    Tq: int                # prefill queries (last Tq positions)
    batch: int = 1         # decode sequences
    modes: tuple = ("flat",)
    beam: int = 64
    n_sink: int = 4
    window: int = 512

    @property
    def q_start(self) -> int:
        return self.T - self.Tq


WORKLOADS = {
    1: Workload(1, "t4k_f32_flat", T=4096, n_comp=64, Hq=4, Hkv=1, D=128, k=256,
                dtype="f32", Tq=4096),
    2: Workload(2, "prefill_t128k_bf16_flat", T=131072, n_comp=1024, Hq=32, Hkv=4,
                D=128, k=2048, dtype="bf16", Tq=131072),
    3: Workload(3, "decode_t1m_b16_bf16_flat", T=1048576, n_comp=4096, Hq=32, Hkv=4,
                D=128, k=2048, dtype="bf16", Tq=1, batch=16),
    4: Workload(4, "prefill_t1m_q8k_bf16_tree", T=1048576, n_comp=1024, Hq=32,
                Hkv=4, D=128, k=2048, dtype="bf16", Tq=8192, modes=("tree", "flat")),
    5: Workload(5, "prefill_t10m_q32k_bf16", T=10_000_000, n_comp=16384, Hq=32,
                Hkv=4, D=128, k=4096, dtype="bf16", Tq=32768, modes=("flat", "tree")),
}


# --------------------------------------------------------------------------
# latent keys and queries (NumPy, host)
# --------------------------------------------------------------------------

def mixture_means(cfg: int, n_comp: int, d: int = 64) -> np.ndarray:
    """Unit-norm component means (fp32), drawn from N(0, I_d) and rescaled."""
    rng = np.random.default_rng(np.random.SeedSequence([SEED, cfg, 0]))
    z = rng.standard_normal((n_comp, d))
    return (z / np.linalg.norm(z, axis=1, keepdims=True)).astype(np.float32)


def component_runs(cfg: int, T: int, n_comp: int, seq: int = 0) -> np.ndarray:
    """Component id per token: runs of U{1..32} tokens, each of a U{0..C-1} component.

    Drawn in fixed batches, so the assignment for T' < T is a prefix of T's.
    """
    rng = np.random.default_rng(np.random.SeedSequence([SEED, cfg, 1, seq]))
    comps, total = [], 0
    while total < T:
        c = rng.integers(0, n_comp, size=65536)
        L = rng.integers(1, 33, size=65536)
        comps.append(np.repeat(c, L))
        total += int(L.sum())
    return np.concatenate(comps)[:T].astype(np.int32)


def _noise_rows(cfg: int, which: int, seq: int, r0: int, r1: int, d: int) -> np.ndarray:
    """Rows [r0, r1) of a fp32 N(0,1) noise matrix drawn in independently seeded chunks."""
    out = np.empty((r1 - r0, d), np.float32)
    c0, c1 = r0 // _ROW_CHUNK, (r1 - 1) // _ROW_CHUNK
    for c in range(c0, c1 + 1):
        rng = np.random.default_rng(np.random.SeedSequence([SEED, cfg, which, seq, c]))
        blk = rng.standard_normal((_ROW_CHUNK, d), dtype=np.float32)
        a, b = max(r0, c * _ROW_CHUNK), min(r1, (c + 1) * _ROW_CHUNK)
        out[a - r0:b - r0] = blk[a - c * _ROW_CHUNK:b - c * _ROW_CHUNK]
    return out


def latent_rows(cfg: int, n_comp: int, comp: np.ndarray, which: str, r0: int, r1: int,
                seq: int = 0, sigma: float = 0.3) -> np.ndarray:
    """Latent keys (which="key") or queries (which="query") for rows [r0, r1), fp32.

    x_t = mu_{c_t} + sigma * eps_t, evaluated in fp32 (one multiply, one add).
    """
    mu = mixture_means(cfg, n_comp)
    eps = _noise_rows(cfg, 2 if which == "key" else 3, seq, r0, r1, mu.shape[1])
    return mu[comp[r0:r1]] + np.float32(sigma) * eps


def latent_query_heads(w: Workload, heads: int, r0: int, r1: int, seq: int = 0,
                       sigma: float = 0.3) -> np.ndarray:
    """H latent query heads per position for rows [r0, r1): [rows, H, 64] fp32.
    Every head of a position is drawn around that position's component mean
    with its own noise; head 0 is the single query latent_inputs returns."""
    comp = component_runs(w.cfg, r1, w.n_comp, seq)
    mu = mixture_means(w.cfg, w.n_comp)
    out = np.empty((r1 - r0, heads, mu.shape[1]), np.float32)
    for h in range(heads):
        eps = _noise_rows(w.cfg, 3 if h == 0 else 16 + h, seq, r0, r1, mu.shape[1])
        out[:, h] = mu[comp[r0:r1]] + np.float32(sigma) * eps
    return out


def latent_inputs(w: Workload, seq: int = 0, T: int | None = None, query_rows=None):
    """(X [T,64] fp32 keys, Y [rows,64] fp32 queries, comp [T]) for one sequence.

    ``query_rows`` defaults to the workload's prefill query range.
    """
    T = w.T if T is None else T
    comp = component_runs(w.cfg, T, w.n_comp, seq)
    X = latent_rows(w.cfg, w.n_comp, comp, "key", 0, T, seq)
    if query_rows is None:
        query_rows = (T - w.Tq, T)
    Y = latent_rows(w.cfg, w.n_comp, comp, "query", query_rows[0], query_rows[1], seq)
    return X, Y, comp


# --------------------------------------------------------------------------
# Philox4x32-10 + Box-Muller (host side, NumPy)
# --------------------------------------------------------------------------
_M0, _M1 = np.uint64(0xD2511F53), np.uint64(0xCD9E8D57)
_W0, _W1 = 0x9E3779B9, 0xBB67AE85
_MASK32 = np.uint64(0xFFFFFFFF)
TENSOR_IDS = {"q": 1, "k": 2, "v": 3}


def philox4x32_10(c0, c1, c2, c3, k0: int, k1: int):
    """Vectorised Philox4x32 with 10 rounds (Salmon et al. 2011, Section 3).

    Each round multiplies words 0 and 2 by the two Philox multipliers (64-bit
    products split into hi/lo halves), swaps and xors the high halves with the
    other two words and the round key; the key is bumped by the Weyl
    constants between rounds.
    """
    c0, c1, c2, c3 = (np.asarray(x, np.uint64) & _MASK32 for x in (c0, c1, c2, c3))
    key0, key1 = k0 & 0xFFFFFFFF, k1 & 0xFFFFFFFF
    for r in range(10):
        if r:
            key0 = (key0 + _W0) & 0xFFFFFFFF
            key1 = (key1 + _W1) & 0xFFFFFFFF
        p0 = _M0 * c0
        p1 = _M1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK32
        c0, c1, c2, c3 = (hi1 ^ c1 ^ np.uint64(key0), lo1,
                          hi0 ^ c3 ^ np.uint64(key1), lo0)
    return c0, c1, c2, c3


def philox_key(cfg: int, tensor: str, seq: int = 0):
    return SEED, (cfg << 16) | (TENSOR_IDS[tensor] << 8) | (seq & 0xFF)


def normal_elements(key, idx: np.ndarray) -> np.ndarray:
    """N(0,1) values (fp64) for flat element indices ``idx`` under Philox ``key``.

    Element e uses counter (e // 4 low, e // 4 high, 0, 0); the four output
    words give two Box-Muller pairs: words (0,1) -> elements 4m, 4m+1 and
    words (2,3) -> elements 4m+2, 4m+3.  u = (w + 0.5) * 2^-32 lies in (0, 1).
    """
    idx = np.asarray(idx, np.uint64)
    m = idx >> np.uint64(2)
    slot = (idx & np.uint64(3)).astype(np.int64)
    w = philox4x32_10(m & _MASK32, m >> np.uint64(32), 0, 0, key[0], key[1])
    wa = np.where(slot < 2, w[0], w[2]).astype(np.float64)
    wb = np.where(slot < 2, w[1], w[3]).astype(np.float64)
    u1 = (wa + 0.5) * 2.0 ** -32
    u2 = (wb + 0.5) * 2.0 ** -32
    r = np.sqrt(-2.0 * np.log(u1))
    th = 6.283185307179586 * u2
    return np.where(slot % 2 == 0, r * np.cos(th), r * np.sin(th))


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp64 to bfloat16, nearest-even, returning the 16-bit patterns."""
    x = np.asarray(x, np.float64)
    m, e = np.frexp(x)                      # x = m * 2^e, 0.5 <= |m| < 1
    e = np.maximum(e, -125)                 # bf16 subnormal quantum is 2^-133
    q = np.ldexp(np.rint(np.ldexp(x, 8 - e)), e - 8)
    return (q.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint32) << np.uint32(16)).view(np.float32)


def normal_rows(w: Workload, tensor: str, rows: np.ndarray, width: int, seq: int = 0,
                row_offset: int = 0):
    """Rows of a [*, width] N(0,1) tensor in the workload's storage dtype.

    Returns float32 values (bf16 values are exactly representable) and, for
    bf16, the raw 16-bit patterns.
    """
    rows = np.asarray(rows, np.int64) + row_offset
    idx = (rows[:, None] * width + np.arange(width)[None, :]).ravel()
    z = normal_elements(philox_key(w.cfg, tensor, seq), idx).reshape(len(rows), width)
    if w.dtype == "f32":
        return z.astype(np.float32), None
    bits = f64_to_bf16_bits(z)
    return bf16_bits_to_f32(bits), bits


# --------------------------------------------------------------------------
# device-side fill (harness-only HIP kernel, same generator definition)
# --------------------------------------------------------------------------
_synth_lib = None


def synth_lib_path() -> str:
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblsa_synth.so")


def _load():
    global _synth_lib
    if _synth_lib is None:
        path = synth_lib_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(path)
        lib.synth_fill_normal.restype = ctypes.c_int
        lib.synth_fill_normal.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                          ctypes.c_uint32, ctypes.c_uint32, ctypes.c_int,
                                          ctypes.c_void_p]
        _synth_lib = lib
    return _synth_lib


def device_fill_normal(ptr: int, n_elems: int, key, elem_offset: int, is_bf16: bool,
                       stream: int = 0) -> None:
    """Fill n_elems device values at ``ptr`` with elements [elem_offset, +n) of the stream."""
    rc = _load().synth_fill_normal(ctypes.c_void_p(ptr), n_elems, elem_offset,
                                   key[0], key[1], 1 if is_bf16 else 0,
                                   ctypes.c_void_p(stream))
    if rc != 0:
        raise RuntimeError(f"synth_fill_normal failed: hip error {rc}")
