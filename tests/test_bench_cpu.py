"""Host logic of bench.py and the input generators, without a GPU: more than one
GPU is refused with a message, the algorithmic byte models match a hand count,
the committed HBM traffic is used only while the kernel source is unchanged, and
seeded workloads are reproducible."""
import hashlib
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
import synth  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""


def test_byte_models_by_hand():
    # CSA: visible entries L // 4 = 1024 and 2048; 4096 completes a block, 8193 does not
    total, keys = bench.csa_bytes([4096, 8193])
    qiw = 64 * 128 + 64 * 4
    assert keys == 128 * (1024 + 2048) + 2 * qiw
    want = keys + 2 * 512 * 580 + 2 * 128 * 1024 + 2 * (2 * 64 * 512 * 2) + (580 + 128 + 4 * 128 * 2)
    assert total == want
    # HCA: 32 and 2 entries, all of them read; 4096 completes a 128-token block
    total, ent = bench.hca_bytes([4096, 300])
    assert ent == 34 * 580
    assert total == ent + 128 * 1024 + 128 * 1024 + 2 * (2 * 64 * 512 * 2) + 580
    # the FP4 key is 64 bytes of codes and 4 of scales
    _, k4 = bench.csa_bytes([4096], key_bytes=bench.KEY_BYTES_FP4, qiw_bytes=bench.QI_W_BYTES_FP4)
    assert k4 == 1024 * 68 + 64 * 68 + 64 * 4


def test_committed_traffic_needs_the_profiled_source(tmp_path):
    src = "long_context_attention_softmax_amd/csrc/indexer.hip"
    sha = hashlib.sha256(open(os.path.join(ROOT, src), "rb").read()).hexdigest()
    good = tmp_path / "good.md"
    good.write_text(f"    kernel_source: {src}\n    kernel_source_sha256: {sha}\n    traffic_bytes_per_launch: 123\n")
    assert bench.committed_traffic(str(good)) == 123
    stale = tmp_path / "stale.md"
    stale.write_text(f"    kernel_source: {src}\n    kernel_source_sha256: {'0' * 64}\n"
                     "    traffic_bytes_per_launch: 123\n")
    assert bench.committed_traffic(str(stale)) is None
    assert bench.committed_traffic(str(tmp_path / "missing.md")) is None
    # several sources: every one must match
    src2 = "long_context_attention_softmax_amd/csrc/pool_block.hpp"
    sha2 = hashlib.sha256(open(os.path.join(ROOT, src2), "rb").read()).hexdigest()
    two = tmp_path / "two.md"
    two.write_text(f"    kernel_source: {src}, {src2}\n    kernel_source_sha256: {sha}, {sha2}\n"
                   "    traffic_bytes_per_launch: 456\n")
    assert bench.committed_traffic(str(two)) == 456
    two.write_text(f"    kernel_source: {src}, {src2}\n    kernel_source_sha256: {sha}, {'1' * 64}\n"
                   "    traffic_bytes_per_launch: 456\n")
    assert bench.committed_traffic(str(two)) is None


def test_seeded_workloads_are_reproducible():
    a, b = synth.make("tiny_f32"), synth.make("tiny_f32")
    for la, lb in zip(a.layers, b.layers):
        for name in ("q", "win", "sink", "gate_w", "gate_b", "q_pos"):
            assert np.array_equal(getattr(la, name), getattr(lb, name)), name
    L1 = synth.gen.ragged_lengths(4, 32, 4096, 1 << 20)
    assert np.array_equal(L1, synth.gen.ragged_lengths(4, 32, 4096, 1 << 20))
    assert L1.min() >= 4096 and L1.max() <= 1 << 20 and len(np.unique(L1)) > 16
