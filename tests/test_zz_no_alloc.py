"""fp4_decode_attention_noalloc (the decode entry point that takes no workspace and allocates
nothing: its split-K partials go to the library's per-GPU scratch array) against
fp4_decode_attention with a caller workspace: the same kernels on the same inputs, so the
outputs must agree bit for bit.  Two calls in a row, the second with a smaller batch and shorter
sequences, so the second call runs on scratch the first one left behind."""
import numpy as np
import pytest

from fp4_kv_cache_amd import workloads as W
from fp4_kv_cache_amd import harness

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "GPU test run without a GPU"
    from fp4_kv_cache_amd import lib
    lib.load()
    return torch


def _noalloc(torch, built, q, bt, seq_lens, zero=None):
    from fp4_kv_cache_amd import lib as L
    batch, hq = q.shape[0], q.shape[1]
    out = torch.full((batch, hq, built.cache.head_dim), float("nan"), dtype=torch.float32, device=q.device)
    dt = L.BF16 if q.dtype == torch.bfloat16 else L.F32
    st = L.fp4_decode_attention_noalloc(built.cache.desc, q.data_ptr(), dt, batch, hq, bt.data_ptr(), bt.shape[1],
                                        seq_lens.data_ptr(), float(W.softmax_scale(built.w)), out.data_ptr(),
                                        zero.data_ptr() if zero is not None else None,
                                        torch.cuda.current_stream().cuda_stream)
    L.check(st, "fp4_decode_attention_noalloc")
    return out


@pytest.mark.parametrize("name", ["qwen3_4b", "qwen3_30b_a3b", "mla", "mla_mxfp4"])
def test_noalloc_matches_the_workspace_entry_point(torch_dev, name):
    torch = torch_dev
    lens = np.array([700, 129, 0, 1500, 64], np.int32)
    w = W.workload(name, batch=len(lens))
    print("noalloc", name, lens.tolist(), flush=True)
    built = harness.build(w, lens=lens)
    q = built.queries()
    scale = W.softmax_scale(w)
    # first call: the whole batch
    zr, zn = (torch.zeros(1, dtype=torch.int32, device=built.device) for _ in range(2))
    ref = built.cache.decode(q, built.bt, built.seq_lens, scale, zero_block_count=zr)
    got = _noalloc(torch, built, q, built.bt, built.seq_lens, zn)
    torch.cuda.synchronize()
    assert torch.equal(got, ref), float((got - ref).abs().max())
    assert int(zr.item()) == int(zn.item())
    # second call: a smaller input (two sequences, shorter) on the scratch the first call left
    lens2 = torch.tensor([300, 100], dtype=torch.int32, device=built.device)
    q2 = q[:2].contiguous()
    bt2 = built.bt[:2].contiguous()
    ref2 = built.cache.decode(q2, bt2, lens2, scale)
    got2 = _noalloc(torch, built, q2, bt2, lens2)
    torch.cuda.synchronize()
    assert torch.equal(got2, ref2), float((got2 - ref2).abs().max())
    assert torch.isfinite(got2).all()
