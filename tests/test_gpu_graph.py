"""Determinism and HIP graph capture of a decode step, through the C ABI.

The library allocates, frees and clears nothing itself, so a caller can capture its calls in
a HIP graph.  A step here is what the bench times: the append of every sequence's newest token
(its position re-appended, which rewrites the same bytes) and fp4_decode_attention.  Two eager
steps must give the same output bytes; the captured step, replayed several times with eager
library work and synchronizations between the replays, must reproduce the eager output bit for
bit on every replay and leave the cache bytes as the eager step left them."""
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


def _step_inputs(torch, built):
    """Persistent device inputs of one append holding the newest token of every non-empty
    sequence (the same rows append_ranges would build)."""
    w, dev = built.w, built.device
    ranges = [(b, int(L) - 1, int(L)) for b, L in enumerate(built.lens) if L > 0]
    seq_ids = np.array([b for b, _, _ in ranges], np.int32)
    pos = np.array([s for _, s, _ in ranges], np.int32)
    slots = np.concatenate([harness.slots_for(built.bt_np[b], np.arange(s, e), w["page"]) for b, s, e in ranges])
    dt = torch.bfloat16 if w["dtype"] == "bf16" else torch.float32
    if w["attn"] == W.GQA:
        k = np.concatenate([np.stack([W.keys(w, b, h, e)[s:e] for h in range(w["hkv"])], axis=1) for b, s, e in ranges])
        v = np.concatenate([np.stack([W.values(w, b, h, e)[s:e] for h in range(w["hkv"])], axis=1) for b, s, e in ranges])
        k = torch.from_numpy(k).to(dt).to(dev).contiguous()
        v = torch.from_numpy(v).to(dt).to(dev).contiguous()
        kr = None
    else:
        k = torch.from_numpy(np.concatenate([W.keys(w, b, 0, e)[s:e][:, None, :] for b, s, e in ranges]))
        k = k.to(dt).to(dev).contiguous()
        v = None
        kr = torch.from_numpy(np.concatenate([W.bf16_bits(W.rope_keys(w, b, e)[s:e]) for b, s, e in ranges])
                              .view(np.int16)).to(dev)
    t = lambda a: torch.from_numpy(a.astype(np.int32)).to(dev)
    return k, v, t(slots), t(seq_ids), t(pos), kr


def _cache_bytes(built):
    return {k: v.clone() for k, v in built.cache.views().items()}


@pytest.mark.parametrize("name", ["qwen3_4b", "qwen3_30b_a3b", "mla", "mla_mxfp4"])
def test_decode_step_graph_replay_is_the_eager_step(torch_dev, name):
    torch = torch_dev
    lens = np.array([700, 129, 0, 1500, 64], np.int32)
    w = W.workload(name, batch=len(lens))
    print("graph", name, lens.tolist(), flush=True)
    built = harness.build(w, lens=lens)
    cache = built.cache
    k, v, slots, seq_ids, pos, kr = _step_inputs(torch, built)
    q = built.queries()
    scale = W.softmax_scale(w)
    B, hq, d = q.shape[0], q.shape[1], cache.head_dim
    ws = torch.empty(max(cache.workspace_bytes(B, hq, built.bt.shape[1] * w["page"]), 4), dtype=torch.uint8,
                     device=built.device)
    out_e = torch.empty((B, hq, d), dtype=torch.float32, device=built.device)
    out_e2 = torch.empty_like(out_e)
    out_g = torch.empty_like(out_e)
    other = torch.empty_like(out_e)

    def step(out):
        cache.append(k, v, slots, seq_ids, pos, kr)
        cache.decode(q, built.bt, built.seq_lens, scale, out=out, workspace=ws)

    # two eager steps: the same bytes
    step(out_e)
    torch.cuda.synchronize()
    snap = _cache_bytes(built)
    step(out_e2)
    torch.cuda.synchronize()
    assert torch.equal(out_e, out_e2), float((out_e - out_e2).abs().max())
    assert torch.isfinite(out_e).all()
    for key, val in _cache_bytes(built).items():
        assert torch.equal(val, snap[key]), "re-appending the newest tokens changed %s" % key

    # the step captured once, replayed three times with eager work in between
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(out_g)
    torch.cuda.synchronize()
    for r in range(3):
        out_g.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), "replay %d: max diff %g" % (r, float((out_g - out_e).abs().max()))
        # eager library work and a synchronization between the replays (shorter sequences)
        cache.decode(q, built.bt, torch.clamp(built.seq_lens - 17, min=0), scale, out=other, workspace=ws)
        torch.cuda.synchronize()
    for key, val in _cache_bytes(built).items():
        assert torch.equal(val, snap[key]), "graph replays changed %s" % key


@pytest.mark.parametrize("name", ["qwen3_4b", "mla"])
def test_noalloc_decode_graph_replay(torch_dev, name):
    """fp4_decode_attention_noalloc (split-K partials in the library's per-GPU scratch array)
    captured in a HIP graph: every replay equals the eager call with a caller workspace."""
    torch = torch_dev
    from fp4_kv_cache_amd import lib as L
    lens = np.array([700, 129, 0, 1500, 64], np.int32)
    w = W.workload(name, batch=len(lens))
    print("graph noalloc", name, lens.tolist(), flush=True)
    built = harness.build(w, lens=lens)
    q = built.queries()
    scale = W.softmax_scale(w)
    B, hq, d = q.shape[0], q.shape[1], built.cache.head_dim
    dt = L.BF16 if q.dtype == torch.bfloat16 else L.F32
    out_g = torch.empty((B, hq, d), dtype=torch.float32, device=built.device)

    def noalloc(out):
        L.check(L.fp4_decode_attention_noalloc(built.cache.desc, q.data_ptr(), dt, B, hq, built.bt.data_ptr(),
                                               built.bt.shape[1], built.seq_lens.data_ptr(), float(scale),
                                               out.data_ptr(), None, torch.cuda.current_stream().cuda_stream),
                "fp4_decode_attention_noalloc")

    ref = built.cache.decode(q, built.bt, built.seq_lens, scale)
    # one eager call before capturing: the first call on a GPU looks up the scratch's address
    eager = torch.empty_like(out_g)
    noalloc(eager)
    torch.cuda.synchronize()
    assert torch.equal(eager, ref), float((eager - ref).abs().max())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        noalloc(out_g)
    torch.cuda.synchronize()
    for r in range(3):
        out_g.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, ref), "replay %d: max diff %g" % (r, float((out_g - ref).abs().max()))
        # eager work on the same scratch between the replays: a shorter batch
        other = torch.empty((2, hq, d), dtype=torch.float32, device=built.device)
        lens2 = torch.tensor([300, 100], dtype=torch.int32, device=built.device)
        q2, bt2 = q[:2].contiguous(), built.bt[:2].contiguous()
        L.check(L.fp4_decode_attention_noalloc(built.cache.desc, q2.data_ptr(), dt, 2, hq, bt2.data_ptr(),
                                               bt2.shape[1], lens2.data_ptr(), float(scale), other.data_ptr(),
                                               None, torch.cuda.current_stream().cuda_stream),
                "fp4_decode_attention_noalloc")
        torch.cuda.synchronize()


@pytest.mark.parametrize("name", ["qwen3_4b", "qwen3_30b_a3b"])
def test_multi_token_decode_graph_replay(torch_dev, name):
    """fp4_decode_attention_multi (two query tokens per sequence, causal) captured in a HIP
    graph: two eager calls give the same bytes and every replay equals them."""
    torch = torch_dev
    lens = np.array([700, 129, 0, 1500, 64], np.int32)
    w = W.workload(name, batch=len(lens))
    print("graph multi", name, lens.tolist(), flush=True)
    built = harness.build(w, lens=lens)
    cache = built.cache
    q = built.queries_multi(2)
    scale = W.softmax_scale(w)
    from fp4_kv_cache_amd import lib as L
    nb = L.fp4_decode_multi_workspace_bytes(cache.desc, q.shape[0], 2, q.shape[2], built.bt.shape[1] * w["page"])
    ws = torch.empty(max(nb, 4), dtype=torch.uint8, device=built.device)
    out_e = cache.decode_multi(q, built.bt, built.seq_lens, scale, workspace=ws)
    out_e2 = cache.decode_multi(q, built.bt, built.seq_lens, scale, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out_e, out_e2)
    assert torch.isfinite(out_e).all()
    out_g = torch.empty_like(out_e)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cache.decode_multi(q, built.bt, built.seq_lens, scale, out=out_g, workspace=ws)
    torch.cuda.synchronize()
    for r in range(3):
        out_g.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), "replay %d: max diff %g" % (r, float((out_g - out_e).abs().max()))
        cache.decode(q[:, -1].contiguous(), built.bt, built.seq_lens, scale, workspace=ws)   # eager work between
        torch.cuda.synchronize()
