"""Host logic of bench.py (no GPU): the single-GPU refusal, the algorithmic byte and flop
counts behind `value` and `roofline`, the choice of the roofline's bound, and the
source-hash gate on the committed counter summaries."""
import hashlib
import os
import subprocess
import sys
import types

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def fake_case(kv_lens, q_len, heads, kv_dtype="e4m3"):
    es = 2 if kv_dtype == "bf16" else 1
    return types.SimpleNamespace(
        kv_lens=torch.tensor(kv_lens, dtype=torch.int32), q_len=q_len, num_heads=heads,
        rows=len(kv_lens) * q_len * heads, kv_bytes=sum(kv_lens) * 576 * es, elem_bytes=es,
        kv_dtype=kv_dtype)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_algorithmic_bytes_headline():
    """H12 q1 B16 128K: 576 B per token row, the q rows, 4 B per block-table entry."""
    by = bench.algorithmic_bytes(fake_case([131072] * 16, 1, 12))
    assert by["kv"] == 16 * 131072 * 576
    assert by["partial_in"] == 16 * 131072 * 576 + 192 * 576 + 16 * 4096 * 4 == 1208332288
    assert by["total"] == by["partial_in"] + 192 * (512 * 2 + 4)
    bf = bench.algorithmic_bytes(fake_case([131072] * 16, 1, 12, "bf16"))
    assert bf["kv"] == 2 * by["kv"] and bf["q"] == 2 * by["q"]


def test_algorithmic_flops_counts_visible_tokens():
    # q = 1: every token, 2 (576 + 512) flop per (row, token)
    assert bench.algorithmic_flops([1000], 1, 12) == 1000 * 12 * 2176
    # q = 8 causal: query j sees L - 8 + j + 1 tokens
    assert bench.algorithmic_flops([100], 8, 2) == sum(100 - 8 + j + 1 for j in range(8)) * 2 * 2176


@pytest.mark.parametrize("lens,q,h,dtype,bound", [
    ([131072] * 16, 1, 12, "e4m3", "hbm"),     # 45 flop/B
    ([131072] * 16, 8, 12, "e4m3", "hbm"),     # ~362 flop/B, ridge 625
    ([100000] * 8, 8, 96, "e4m3", "mfma"),     # ~2900 flop/B
    ([1 << 20], 8, 12, "bf16", "hbm"),         # ~181 flop/B, ridge 312
    ([1 << 20], 8, 96, "bf16", "mfma"),
])
def test_roofline_bound(lens, q, h, dtype, bound):
    case = fake_case(lens, q, h, dtype)
    by = bench.algorithmic_bytes(case)
    r = bench.roofline("no_such_workload", case, by, 100.0)
    assert r["bound"] == bound and r["traffic"] is None
    if bound == "hbm":
        assert r["unit"] == "GB/s" and r["peak"] == 8000.0
        assert r["achieved"] == pytest.approx(by["partial_in"] / 100e-6 / 1e9, abs=0.1)
    else:
        fl = bench.algorithmic_flops(lens, q, h)
        assert r["unit"] == "TFLOP/s" and r["peak"] == (5000.0 if dtype == "e4m3" else 2500.0)
        assert r["achieved"] == pytest.approx(fl / 100e-6 / 1e12, abs=0.01)
    assert r["frac"] == pytest.approx(r["achieved"] / r["peak"], abs=1e-4)
    assert r["kernel"] == bench.dominant_kernel(dtype, q * h)[0]


def test_traffic_only_while_the_source_hash_matches(tmp_path, monkeypatch):
    (tmp_path / "profiles").mkdir()
    csrc = tmp_path / "decode_attention_gather_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "k.hip").write_bytes(b"kernel source")
    sha = hashlib.sha256(b"kernel source").hexdigest()
    (tmp_path / "profiles" / "k_kernel_w.md").write_text(
        f"# summary\n\n    traffic_bytes_per_launch: 1234\n    kernel_source_sha256: {sha}\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.profiled_traffic("w", "k_kernel", "k.hip") == 1234
    (csrc / "k.hip").write_bytes(b"kernel source, edited")
    assert bench.profiled_traffic("w", "k_kernel", "k.hip") is None
    assert bench.profiled_traffic("other", "k_kernel", "k.hip") is None


@pytest.mark.parametrize("lens, q, h", [
    ([2048], 1, 12),            # small: every row
    ([1048576], 1, 12),         # one long request: every row, 12 x 1M row-tokens
    ([131072] * 16, 8, 12),     # 1536 rows: a sample within the row-token budget
    ([1048576] + [4096] * 7, 8, 12),
])
def test_oracle_sample_is_bounded(lens, q, h):
    case = fake_case(lens, q, h, "e4m3")
    n = bench.oracle_rows(case)
    assert 1 <= n <= case.rows
    assert n == case.rows or n == 16 or n * max(lens) <= bench.ORACLE_ROW_TOKENS
    assert n >= min(16, case.rows)
