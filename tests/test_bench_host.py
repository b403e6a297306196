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

KERNEL = "k_near_attn<8> + k_attn_bf16<1, 4, true>"
WORKLOAD = "prefill_t128k_bf16_flat"
SOURCES = ["sparse_attention_indexing_amd/csrc/lsa_dense.hip",
           "sparse_attention_indexing_amd/csrc/lsa_attn.hip"]


def test_workload_names():
    assert bench.workload_name("prefill_t1m_q8k_bf16_flat", "tree") == "prefill_t1m_q8k_bf16_tree"
    assert bench.workload_name("prefill_t128k_bf16_flat", "flat") == "prefill_t128k_bf16_flat"
    assert bench.workload_name("decode_x", "tree") == "decode_x"


def test_attention_kernel_names():
    # the 128K workload's caches take one workgroup per (row, KV head), the 1M
    # and 10M ones one workgroup per row; the prefill attention runs the
    # near-set kernel before each gather
    w2, w4, w5 = S.WORKLOADS[2], S.WORKLOADS[4], S.WORKLOADS[5]
    assert bench.attention_kernel_name(lsa, w2, 1, w2.T) == "k_attn_bf16<1, 4>"
    assert bench.attention_kernel_name(lsa, w2, 1, w2.T, True) == KERNEL
    assert bench.attention_kernel_name(lsa, w4, 1, w4.T) == "k_attn_bf16<4, 4>"
    assert bench.attention_kernel_name(lsa, w5, 1, w5.T, True) == "k_attn_bf16<4, 4, true>"
    assert bench.attention_kernel_name(lsa, S.WORKLOADS[1], 1, 4096) == "k_attn_f32"


def _summary(root, kernel, sources, rows, digest=None):
    import hashlib
    os.makedirs(os.path.join(root, "profiles"), exist_ok=True)
    blob = b"".join(open(os.path.join(ROOT, f), "rb").read() for f in sources)
    digest = digest or hashlib.sha256(blob).hexdigest()[:16]
    stem = "attention_prefill" if "+" in kernel else kernel.split("<")[0]
    for f in sources:
        os.makedirs(os.path.dirname(os.path.join(root, f)), exist_ok=True)
        with open(os.path.join(root, f), "wb") as out:
            out.write(open(os.path.join(ROOT, f), "rb").read())
    with open(os.path.join(root, "profiles", f"{stem}.{WORKLOAD}.traffic.md"), "w") as out:
        out.write(f"# x\n\nkernel: {kernel}\ntraffic_bytes_per_launch: 1.5e9\n"
                  f"rows_per_launch: {rows}\nkernel_source: {', '.join(sources)}\n"
                  f"kernel_source_sha256_16: {digest}\n")


def test_traffic_is_taken_only_for_the_summarised_kernel_and_source(tmp_path):
    rows = lsa.attention_launch_rows()
    root = str(tmp_path)
    _summary(root, KERNEL, SOURCES, rows)
    assert bench.measured_traffic(KERNEL, WORKLOAD, rows, root) == 1.5e9
    # any other instance, launch size or workload has no figure
    assert bench.measured_traffic("k_attn_bf16<1, 4>", WORKLOAD, rows, root) is None
    assert bench.measured_traffic(KERNEL, WORKLOAD, 2 * rows, root) is None
    assert bench.measured_traffic(KERNEL, "prefill_t10m_q32k_bf16_flat", rows, root) is None
    # a summary taken on another source has no figure
    _summary(root, KERNEL, SOURCES, rows, digest="0123456789abcdef")
    assert bench.measured_traffic(KERNEL, WORKLOAD, rows, root) is None


def test_committed_traffic_if_any_matches_the_committed_kernel():
    # a committed summary for the benchmark's kernel pair gives a figure only
    # when it was taken on the sources in this tree
    rows = lsa.attention_launch_rows()
    path = os.path.join(ROOT, "profiles", f"attention_prefill.{WORKLOAD}.traffic.md")
    t = bench.measured_traffic(KERNEL, WORKLOAD, rows)
    if os.path.exists(path) and t is None:
        pytest.skip("the committed traffic summary predates the current kernel sources")
    assert t is None or t > 1e8
