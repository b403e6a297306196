"""GPU parity of the dense (and banded) causal attention baseline, through
the C ABI: every query row against the oracle's attention over the keys
[max(0, p - band + 1), p] (band unbounded: dense causal attention, which the
oracle's pins tie to torch SDPA with is_causal=True), within 2e-2 max-abs in
bf16; ragged row counts, key counts that are not a multiple of the 16-key
tile, every supported GQA group size, and the 128K workload's shape."""
import sys

import numpy as np
import pytest
import torch

import lsa_synth as S
import sparse_attention_indexing_amd as lsa
from oracle import lsa_oracle as O
from parity_util import attention_from_rows, bf16_tensor, device_normal, host_rows

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lsa.lib()


def _bf16_normal(rng, shape):
    u = rng.standard_normal(shape).astype(np.float32).view(np.uint32)
    bits = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    vals = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return vals, bits


@pytest.mark.parametrize("Hq,Hkv,band", [(32, 4, None), (32, 4, 512), (32, 4, 1), (16, 1, None),
                                         (8, 2, 37), (32, 8, None), (4, 4, None), (32, 2, 300)])
def test_dense_attention_against_oracle(Hq, Hkv, band):
    say(f"case: dense attention Hq={Hq} Hkv={Hkv} band={band}")
    D, Tk, q_start = 128, 2999, 1700          # 1,299 rows: ragged workgroup tiles
    Tq = Tk - q_start
    rng = np.random.default_rng(Hq * 7 + Hkv + (band or 0))
    q, qb = _bf16_normal(rng, (Tq, Hq, D))
    k, kb = _bf16_normal(rng, (Tk, Hkv, D))
    v, vb = _bf16_normal(rng, (Tk, Hkv, D))
    out = lsa.dense_attention(bf16_tensor(qb).cuda(), bf16_tensor(kb).cuda(), bf16_tensor(vb).cuda(),
                              q_start, band=band)
    torch.cuda.synchronize()
    out = out.float().cpu().numpy()
    rows = np.unique(np.concatenate([[0, 1, 15, 16, 17, Tq - 1, Tq - 2], np.arange(0, Tq, 97)]))
    err = 0.0
    for r in rows:
        p = q_start + int(r)
        lo = 0 if band is None else max(0, p - band + 1)
        idx = np.arange(lo, p + 1)
        err = max(err, float(np.abs(out[r] - O.attention_query(q[r], k, v, idx, len(idx))).max()))
    say(f"max abs err {err:.3g} over {len(rows)} rows")
    assert err <= 2e-2


def test_dense_attention_whole_prefill_small():
    """q_start = 0: every row of a 600-token prefill, the first rows attending
    to a single key."""
    say("case: dense attention, whole prefill of 600 tokens")
    rng = np.random.default_rng(3)
    D, T, Hq, Hkv = 128, 600, 8, 1
    q, qb = _bf16_normal(rng, (T, Hq, D))
    k, kb = _bf16_normal(rng, (T, Hkv, D))
    v, vb = _bf16_normal(rng, (T, Hkv, D))
    out = lsa.dense_attention(bf16_tensor(qb).cuda(), bf16_tensor(kb).cuda(), bf16_tensor(vb).cuda(), 0)
    torch.cuda.synchronize()
    out = out.float().cpu().numpy()
    err = max(float(np.abs(out[p] - O.attention_query(q[p], k, v, np.arange(p + 1), p + 1)).max())
              for p in range(T))
    say(f"max abs err {err:.3g} over {T} rows")
    assert err <= 2e-2


def test_dense_attention_128k_workload():
    """The 128K prefill's Q/K/V (device generator): dense causal attention of
    every row; sampled rows against the oracle."""
    say("case: dense attention, T = 131072")
    w = S.WORKLOADS[2]
    Q = device_normal(w, "q", (w.Tq, w.Hq, w.D))
    K = device_normal(w, "k", (w.T, w.Hkv, w.D))
    V = device_normal(w, "v", (w.T, w.Hkv, w.D))
    out = lsa.dense_attention(Q, K, V, 0)
    torch.cuda.synchronize()
    rows = [0, 517, 70001, w.T - 1]
    q_rows = host_rows(w, "q", rows, w.Hq * w.D)
    out_h = out.float().cpu().numpy()
    err = 0.0
    for i, p in enumerate(rows):
        idx = np.arange(p + 1, dtype=np.int32)
        err = max(err, float(np.abs(out_h[p] - attention_from_rows(w, q_rows[i], idx, p + 1)).max()))
    say(f"max abs err {err:.3g} over {len(rows)} rows")
    assert err <= 2e-2
