"""Host logic of bench.py (no GPU): the measured-traffic figure in its roofline
object is taken from the committed counter summary only for the kernel
instance, kernel source and launch size that the summary was taken on."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import lsa_synth as S  # noqa: E402
import sparse_attention_indexing_amd as lsa  # noqa: E402

KERNEL, WORKLOAD = "k_attn_bf16<1, 4>", "prefill_t128k_bf16_flat"


def test_workload_names():
    assert bench.workload_name("prefill_t1m_q8k_bf16_flat", "tree") == "prefill_t1m_q8k_bf16_tree"
    assert bench.workload_name("prefill_t128k_bf16_flat", "flat") == "prefill_t128k_bf16_flat"
    assert bench.workload_name("decode_x", "tree") == "decode_x"


def test_attention_kernel_names():
    # the 128K workload's caches take one workgroup per (row, KV head), the 1M
    # and 10M ones one workgroup per row
    assert bench.attention_kernel_name(lsa, S.WORKLOADS[2], 1, S.WORKLOADS[2].T) == KERNEL
    assert bench.attention_kernel_name(lsa, S.WORKLOADS[4], 1, S.WORKLOADS[4].T) == "k_attn_bf16<4, 4>"
    assert bench.attention_kernel_name(lsa, S.WORKLOADS[5], 1, S.WORKLOADS[5].T) == "k_attn_bf16<4, 4>"
    assert bench.attention_kernel_name(lsa, S.WORKLOADS[1], 1, 4096) == "k_attn_f32"


def test_committed_traffic_matches_the_committed_kernel():
    # the summary under profiles/ was taken on the kernel source in this tree
    # with the library's launch size
    rows = lsa.attention_launch_rows()
    t = bench.measured_traffic(KERNEL, WORKLOAD, rows)
    assert t is not None and t > 1e8
    # any other instance, launch size or workload has no figure
    assert bench.measured_traffic("k_attn_bf16<4, 4>", WORKLOAD, rows) is None
    assert bench.measured_traffic(KERNEL, WORKLOAD, 2 * rows) is None
    assert bench.measured_traffic(KERNEL, "prefill_t10m_q32k_bf16_flat", rows) is None
