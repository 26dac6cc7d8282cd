"""GPU parity of the BF16-KV comparison path (bf16kv_append, bf16_decode_attention) against
oracle/bf16attn.py: cache bytes bit-exact (bf16 of the inputs, nearest even, in the library's
layout), decode rows within 1e-3 of the row norm; the error against unquantized fp64 attention
is printed beside the FP4 path's."""
import numpy as np
import pytest

from fp4_kv_cache_amd import workloads as W
from fp4_kv_cache_amd import harness
from oracle import attention as A
from oracle import bf16attn as BA
from _gpu import say

pytestmark = pytest.mark.gpu
TOL = 1e-3


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "GPU test run without a GPU"
    from fp4_kv_cache_amd import lib
    lib.load()
    return torch


def _bits(x):
    return (BA.bf16(x).view(np.uint32) >> 16).astype(np.uint16)


def check_bf16_cache(built):
    w = built.w
    v = {k: t.cpu().numpy().view(np.uint16) for k, t in built.cache.views().items()}
    P = w["page"]
    for b in range(w["batch"]):
        L = int(built.lens[b])
        if L == 0:
            continue
        pos = np.arange(L)
        pages, offs = built.bt_np[b][pos // P], pos % P
        for h in range(w["hkv"]):
            gk = v["k"][pages, h, offs, :]
            gv = v["v"][pages, h, :, offs]
            assert np.array_equal(gk, _bits(W.keys(w, b, h, L))), (b, h, "k")
            assert np.array_equal(gv, _bits(W.values(w, b, h, L))), (b, h, "v")


def compare_bf16(built, tol=TOL):
    import torch
    w = built.w
    g = w["hq"] // w["hkv"]
    q = built.queries()
    out = built.cache.decode(q, built.bt, built.seq_lens, W.softmax_scale(w))
    torch.cuda.synchronize()
    qn, out = q.float().cpu().numpy(), out.cpu().numpy()
    worst, num, den = 0.0, 0.0, 0.0
    for b in range(w["batch"]):
        L = int(built.lens[b])
        for h in range(w["hkv"]):
            got = out[b, h * g:(h + 1) * g]
            assert np.all(np.isfinite(got)), (b, h)
            if L == 0:
                assert not np.any(got), (b, h)
                continue
            rows = qn[b, h * g:(h + 1) * g]
            K, V = W.keys(w, b, h, L), W.values(w, b, h, L)
            exp = BA.bf16_attention(rows, K, V, W.softmax_scale(w), L=L)
            e = float(np.max(A.row_rel_err(got, exp)))
            worst = max(worst, e)
            assert e <= tol, "seq %d kv head %d: max row error %.3g" % (b, h, e)
            ref = A.reference_attention(rows, K, V, W.softmax_scale(w))
            num += float(np.sum((got - ref) ** 2))
            den += float(np.sum(ref ** 2))
    agg = (num / den) ** 0.5 if den else 0.0
    say("bf16: max err vs oracle %.3g, error vs fp64 attention over all rows %.4f" % (worst, agg))
    assert agg < 0.05
    return worst, agg


@pytest.mark.parametrize("name,hq,page", [("qwen3_4b", 8, 64), ("qwen3_4b", 32, 16), ("qwen3_30b_a3b", 32, 256),
                                          ("qwen3_30b_a3b", 64, 32), ("tiny", 16, 128), ("qwen3_4b", 16, 64)])
def test_bf16_decode_matches_oracle(torch_dev, name, hq, page):
    """Ragged lengths around the 64-token softmax tile and the 128-token partition tile
    (0, 1, 63, 64, 65, 129, 700, 2000); one to sixteen query heads per KV head; every page
    size; bf16 and fp32 (tiny) inputs."""
    lens = np.array([1, 63, 0, 64, 65, 129, 700, 2000], np.int32)
    w = W.workload(name, batch=len(lens), hq=hq, page=page)
    say("bf16 decode %s hq=%d page=%d" % (name, hq, page), lens.tolist())
    built = harness.build_bf16(w, lens=lens)
    check_bf16_cache(built)
    compare_bf16(built)


def test_bf16_decode_long_shares(torch_dev, monkeypatch):
    """One share streaming a sequence past the page-id window (FP4KV_MAX_SHARES=1)."""
    monkeypatch.setenv("FP4KV_MAX_SHARES", "1")
    lens = np.array([9000, 3], np.int32)
    w = W.workload("tiny", batch=len(lens), page=16)
    say("bf16 decode long share", lens.tolist())
    built = harness.build_bf16(w, lens=lens)
    compare_bf16(built)
