"""Build a prefilled paged FP4 cache for a synthetic workload on the GPU.

Host plumbing only: draws the workload's inputs (``workloads``), moves them to
the device with torch and feeds them through the library's ``kv_quant_append``;
all quantization happens in the HIP kernels.
"""
import numpy as np

from . import workloads as W
from .lib import PagedFP4Cache, PagedBF16Cache, GQA, MLA


def _dev(x, w, torch, device):
    t = torch.from_numpy(np.ascontiguousarray(x))
    if w["dtype"] == "bf16":
        t = t.to(torch.bfloat16)
    return t.to(device)


class Built:
    """A prefilled cache with the workload's page table, lengths and calibration."""

    def __init__(self, w, cache, bt, lens, calib, device):
        import torch
        self.w, self.cache, self.lens, self.calib = w, cache, lens, calib
        self.bt_np = bt
        self.bt = torch.from_numpy(bt).to(device)
        self.seq_lens = torch.from_numpy(lens.astype(np.int32)).to(device)
        self.device = device

    def queries(self):
        import torch
        q = np.stack([W.queries(self.w, b) for b in range(self.w["batch"])])
        if self.w["attn"] == MLA:
            qr = np.stack([W.rope_queries(self.w, b) for b in range(self.w["batch"])])
            q = np.concatenate([q, qr], axis=-1)
        return _dev(q, self.w, torch, self.device)

    def queries_multi(self, n):
        """[batch, n, Hq, d] queries of every sequence's n newest tokens (GQA)."""
        import torch
        q = np.stack([W.queries_multi(self.w, b, n) for b in range(self.w["batch"])])
        return _dev(q, self.w, torch, self.device)


def slots_for(bt_row, positions, P):
    positions = np.asarray(positions, np.int64)
    return (bt_row[positions // P].astype(np.int64) * P + positions % P).astype(np.int32)


def build(w, lens=None, copy=0, device="cuda", stop=None, workers=8, calib=None):
    """Allocate the cache for workload ``w`` and append every sequence's context.

    ``stop`` (optional int array) appends only the first stop[b] tokens of each
    sequence; the rest can be appended later with ``append_range``.  The keys
    and values of the tokens left out are kept in ``built.tail[b]`` (GQA).
    ``calib`` replaces the workload's calibration (k_smooth_inv, q_smooth, G_K, G_V).
    """
    import torch
    lens = W.seq_lens(w) if lens is None else np.asarray(lens, np.int32)
    bt, num_pages = W.page_table(w, lens, copy)
    ksi, qs, gk, gv = W.calibration(w) if calib is None else calib
    attn = w["attn"]
    cache = PagedFP4Cache(w["fmt"], attn, num_pages, w["page"], w["hkv"], w["d"], w["batch"],
                          ksi, qs, gk if w["fmt"] == 0 else None,
                          gv if (w["fmt"] == 0 and attn == GQA) else None,
                          rope_dim=w["rope"], device=device)
    built = Built(w, cache, bt, lens, (ksi, qs, gk, gv), device)
    stop = lens if stop is None else np.asarray(stop)
    built.tail = {}
    for b in range(w["batch"]):
        built.tail[b] = append_range(built, b, 0, int(stop[b]), workers=workers, gen_end=int(lens[b]))
    return built


def append_range(built, b, start, end, workers=8, gen_end=None):
    """Append positions [start, end) of sequence b in one kv_quant_append call.

    With ``gen_end`` > end the inputs are drawn up to gen_end and the rows
    [end, gen_end) are returned as (keys, values) [n, Hkv, d] float32 (GQA).
    """
    import torch
    w, cache, dev = built.w, built.cache, built.device
    n = end - start
    gen_end = end if gen_end is None else max(gen_end, end)
    if n <= 0 and gen_end == end:
        return None
    pos = np.arange(start, end, dtype=np.int32)
    slots = slots_for(built.bt_np[b], pos, w["page"])
    tail = None
    if w["attn"] == GQA:
        ks = W.parallel_map(lambda h: W.keys(w, b, h, gen_end)[start:], range(w["hkv"]), workers)
        vs = W.parallel_map(lambda h: W.values(w, b, h, gen_end)[start:], range(w["hkv"]), workers)
        kall, vall = np.stack(ks, axis=1), np.stack(vs, axis=1)
        tail = (kall[n:], vall[n:])
        if n <= 0:
            return tail
        k = _dev(kall[:n], w, torch, dev)
        v = _dev(vall[:n], w, torch, dev)
        kr = None
    else:
        if n <= 0:
            return None
        k = _dev(W.keys(w, b, 0, end)[start:end][:, None, :], w, torch, dev)
        v = None
        kr = torch.from_numpy(W.bf16_bits(W.rope_keys(w, b, end)[start:end]).view(np.int16)).to(dev)
    cache.append(k, v, torch.from_numpy(slots).to(dev), torch.full((n,), b, dtype=torch.int32, device=dev),
                 torch.from_numpy(pos).to(dev), kr)
    return tail


def append_step(built, pos):
    """One kv_quant_append call holding token pos[b] of every sequence b with pos[b] >= 0
    (a decode step: one new token per sequence, in sequence order)."""
    append_ranges(built, [(b, int(pos[b]), int(pos[b]) + 1) for b in range(built.w["batch"]) if pos[b] >= 0])


def append_ranges(built, ranges):
    """One kv_quant_append call holding positions [start, end) of each (b, start, end) in
    `ranges` (sequences in increasing order, each at most once)."""
    import torch
    w, cache, dev = built.w, built.cache, built.device
    ranges = [(b, s, e) for b, s, e in ranges if e > s]
    if not ranges:
        return
    seq_ids = np.concatenate([np.full(e - s, b, np.int32) for b, s, e in ranges])
    p = np.concatenate([np.arange(s, e, dtype=np.int32) for _, s, e in ranges])
    slots = np.concatenate([slots_for(built.bt_np[b], np.arange(s, e), w["page"]) for b, s, e in ranges])
    if w["attn"] == GQA:
        k = np.concatenate([np.stack([W.keys(w, b, h, e)[s:e] for h in range(w["hkv"])], axis=1)
                            for b, s, e in ranges])
        v = np.concatenate([np.stack([W.values(w, b, h, e)[s:e] for h in range(w["hkv"])], axis=1)
                            for b, s, e in ranges])
        k, v, kr = _dev(k, w, torch, dev), _dev(v, w, torch, dev), None
    else:
        k = _dev(np.concatenate([W.keys(w, b, 0, e)[s:e][:, None, :] for b, s, e in ranges]), w, torch, dev)
        v = None
        kr = torch.from_numpy(np.concatenate([W.bf16_bits(W.rope_keys(w, b, e)[s:e]) for b, s, e in ranges])
                              .view(np.int16)).to(dev)
    cache.append(k, v, torch.from_numpy(slots.astype(np.int32)).to(dev), torch.from_numpy(seq_ids).to(dev),
                 torch.from_numpy(p).to(dev), kr)


def build_bf16(w, lens=None, copy=0, device="cuda", workers=8):
    """The same workload's keys and values in the BF16 comparison cache (GQA workloads):
    every sequence appended with bf16kv_append, the same page table as ``build``."""
    import torch
    assert w["attn"] == GQA
    lens = W.seq_lens(w) if lens is None else np.asarray(lens, np.int32)
    bt, num_pages = W.page_table(w, lens, copy)
    cache = PagedBF16Cache(num_pages, w["page"], w["hkv"], device=device)
    built = Built(w, cache, bt, lens, None, device)
    for b in range(w["batch"]):
        L = int(lens[b])
        if L == 0:
            continue
        ks = W.parallel_map(lambda h: W.keys(w, b, h, L), range(w["hkv"]), workers)
        vs = W.parallel_map(lambda h: W.values(w, b, h, L), range(w["hkv"]), workers)
        slots = slots_for(bt[b], np.arange(L), w["page"])
        cache.append(_dev(np.stack(ks, axis=1), w, torch, device), _dev(np.stack(vs, axis=1), w, torch, device),
                     torch.from_numpy(slots).to(device))
    return built
