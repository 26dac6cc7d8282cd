"""Host-side arithmetic of bench.py (no GPU): the bytes and flops it divides by, the matrix peak
of the MLA roofline, and the single-GPU contract."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from fp4_kv_cache_amd import workloads as W  # noqa: E402


def test_kv_bytes_per_token_head():
    # GQA: K and V codes (64 B each) plus one scale byte per block of 16 (NVFP4) or 32 (MXFP4)
    assert bench.kv_bytes_per_token_head(W.workload("qwen3_4b")) == 64 + 8 + 64 + 8
    assert bench.kv_bytes_per_token_head(W.workload("qwen3_30b_a3b")) == 64 + 4 + 64 + 4
    # MLA: 256 B of latent codes, one scale per 16 x 16 (32 x 32) tile, 64 bf16 rope values
    assert bench.kv_bytes_per_token_head(W.workload("mla")) == 256 + 2 + 128
    assert bench.kv_bytes_per_token_head(W.workload("mla_mxfp4")) == 256 + 0.5 + 128


def test_qwen3_4b_bytes_per_step():
    w = W.workload("qwen3_4b")
    lens = W.seq_lens(w)
    assert int(lens.sum()) * w["hkv"] * bench.kv_bytes_per_token_head(w) == 603979776


def test_mla_flops_per_step():
    w = W.workload("mla")
    # Q1 and Q2 rows of 128 heads over the 512 latent channels, the rope part once per head
    # (64 channels, unquantized), P.V over the 512 latent channels
    assert bench.mla_flops_per_token(w) == 2 * 256 * 512 + 2 * 128 * 64 + 2 * 128 * 512
    lens = W.seq_lens(w)
    total = float(lens.sum()) * bench.mla_flops_per_token(w)
    assert 214.7e9 < total < 214.8e9        # 32 x 16384 tokens: 214.7 GFLOP per step
    assert bench.FP4_MFMA_PEAK_TFLOPS == 10100.0


def test_more_than_one_gpu_exits():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in r.stderr or "one GPU" in r.stdout
