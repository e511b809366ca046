"""Host logic of bench.py and accounting.py (CPU only): the one-GPU contract, the FLOP and
byte counts the bench line is built from, and the rule that a stored traffic figure is used
only while the kernel's sources are unchanged (otherwise the line reports it as null)."""
import json
import os
import subprocess
import sys
import types

import pytest

from block_sparse_linear_pool_amd import accounting as acc

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, REPO)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(REPO, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and not r.stdout


def test_counts_of_the_12_head_workload():
    """B = 1, H = 12, N = 32768, 15 of 512 key blocks kept: 4 B H N^2 d = 6.597 TFLOP of dense
    attention; 4 * 128 * 64 * d FLOP for each of the 12 * 256 * 15 = 46 080 kept pairs =
    193.3 GFLOP; 97.07 % sparsity."""
    p = acc.Problem(1, 12, 32768, 15)
    assert p.pairs == 46080
    assert acc.full_attention_flops(p) == 4 * 12 * 32768 ** 2 * 128
    assert round(acc.full_attention_flops(p) / 1e12, 3) == 6.597
    assert acc.sparse_flops(p) == 4 * 128 * 64 * 128 * 46080
    assert round(acc.sparse_flops(p) / 1e9, 1) == 193.3
    assert acc.kernel_flops(p, "attn") == acc.sparse_flops(p)
    assert round(p.sparsity, 4) == 0.9707
    # minimum bytes: Q, K, V (bf16) once, K again, O in fp32, bf16 h_j^T and fp32 z_j written
    # and read once
    E = 12 * 32768 * 128
    assert acc.call_min_bytes(p) == 4 * E * 2 + E * 4 + 2 * 12 * 512 * (128 * 128 * 2 + 128 * 4)
    assert round(acc.call_min_bytes(p) / 1e9, 3) == 1.013


def test_counts_of_the_40_head_workload():
    """B = 1, H = 40, N = 75648, 59 of 1182 key blocks kept: 117.2 TFLOP dense, 5.85 TFLOP in
    the sparse branch."""
    p = acc.Problem(1, 40, 75648, 59)
    assert round(acc.full_attention_flops(p) / 1e12, 1) == 117.2
    assert round(acc.sparse_flops(p) / 1e12, 2) == 5.85


def test_whole_call_fraction_takes_the_larger_bound():
    p = acc.Problem(1, 12, 32768, 15)
    t_hbm = acc.call_min_bytes(p) / 8.0e12
    t_mfma = acc.sparse_flops(p) / 5.0e15
    assert t_hbm > t_mfma   # this workload is HBM-bound as a whole
    assert acc.whole_call_frac(p, 2 * t_hbm) == pytest.approx(0.5)
    q = acc.Problem(1, 12, 32768, 512)   # everything kept: the matrix work dominates
    t = acc.sparse_flops(q) / 5.0e15
    assert acc.whole_call_frac(q, 4 * t) == pytest.approx(0.25)


def test_router_counts_follow_where_each_product_is_formed():
    """project forms B = Kbar_s Wk and A = Qbar Wq ((N/64 + N/128) d^2 MACs per head);
    score_topk the logits ((N/128)(N/64) d MACs per head)."""
    p = acc.Problem(1, 12, 32768, 15)
    assert acc.kernel_flops(p, "project") == 2 * 12 * (512 + 256) * 128 * 128
    assert acc.kernel_flops(p, "score_topk") == 2 * 12 * 256 * 512 * 128


def test_stored_traffic_is_used_only_for_unchanged_sources(tmp_path):
    w = types.SimpleNamespace(name="wan13b_480p_N32768")
    rec = {"kernel": "attn", "workload": w.name, "keep_frac": 0.03,
           "source_sha256": bench.kernel_source_hash("attn"), "bytes_per_launch": 1234}
    path = tmp_path / "t.json"
    args = types.SimpleNamespace(traffic=str(path))
    path.write_text(json.dumps(rec))
    assert bench.stored_traffic(args, "attn", w, 0.03) == 1234
    assert bench.stored_traffic(args, "attn", w, 0.05) is None           # another keep
    assert bench.stored_traffic(args, "kv_prep", w, 0.03) is None        # another kernel
    path.write_text(json.dumps(dict(rec, source_sha256="0" * 16)))
    assert bench.stored_traffic(args, "attn", w, 0.03) is None           # sources changed
    # the hash covers the kernel's own source and the shared header
    assert bench.kernel_source_hash("attn") != bench.kernel_source_hash("kv_prep")
    assert bench.kernel_source_hash("bwd_kv") == bench.kernel_source_hash("bwd_q")


def test_cpu_sample_text():
    w = types.SimpleNamespace(H=12)
    assert bench.heads_text([0, 1, 2], w) == "heads 0-2 of 12"
    assert bench.heads_text(list(range(12)) + [0, 1], w) == "heads 0-11 of 12 (14 head passes)"
