"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Append: cache bytes bit-exact.  Decode: max |out - oracle| / ||oracle row||_2 <= 1e-3
per row; the error against unquantized fp64 attention is printed.
"""
import numpy as np
import pytest

from fp4_kv_cache_amd import workloads as W
from fp4_kv_cache_amd import harness
from _gpu import say, check_gqa_cache, check_mla_cache, compare_gqa, compare_gqa_multi, compare_mla

pytestmark = pytest.mark.gpu
TOL = 1e-3


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "GPU test run without a GPU"
    from fp4_kv_cache_amd import lib
    lib.load()
    return torch


def test_append_tiny_nvfp4_bitexact(torch_dev):
    w = W.workload("tiny")
    say("append tiny nvfp4 page16 L=4096")
    built = harness.build(w)
    check_gqa_cache(built)


def test_append_mxfp4_ragged_bitexact(torch_dev):
    w = W.workload("qwen3_30b_a3b", batch=3)
    lens = np.array([100, 33, 700], np.int32)
    say("append mxfp4 ragged", lens.tolist())
    built = harness.build(w, lens=lens)
    check_gqa_cache(built)


def test_append_incremental_tail_requant(torch_dev):
    """Prefill part of each sequence, then append in uneven chunks (1, 5, 17, ... tokens);
    the cache must equal the one-shot quantization of the final sequences."""
    for name in ("qwen3_4b", "qwen3_30b_a3b"):
        w = W.workload(name, batch=2)
        lens = np.array([300, 97], np.int32)
        stop = np.array([150, 37], np.int32)
        say("append incremental", name, lens.tolist(), stop.tolist())
        built = harness.build(w, lens=lens, stop=stop)
        rng = np.random.default_rng(5)
        for b in range(2):
            p = int(stop[b])
            while p < lens[b]:
                n = int(min(lens[b] - p, rng.choice([1, 1, 2, 5, 17, 40])))
                harness.append_range(built, b, p, p + n)
                p += n
        check_gqa_cache(built)


@pytest.mark.parametrize("name", ["qwen3_4b", "qwen3_30b_a3b", "mla", "mla_mxfp4"])
def test_append_decode_steps(torch_dev, name):
    """Decode-step appends: after a prefill, every call adds one token to each sequence
    (three sequences at different offsets inside their blocks), across block and page
    boundaries; the cache must equal the one-shot quantization of the final sequences."""
    stop = np.array([40, 63, 95], np.int32)
    lens = stop + 40
    w = W.workload(name, batch=len(lens))
    say("append decode steps", name, stop.tolist(), lens.tolist())
    built = harness.build(w, lens=lens, stop=stop)
    for k in range(40):
        harness.append_step(built, stop + k)
    if w["attn"] == 0:
        check_gqa_cache(built)
    else:
        check_mla_cache(built)


@pytest.mark.parametrize("name", ["qwen3_4b", "qwen3_30b_a3b", "mla", "mla_mxfp4"])
def test_append_mixed_chunks_one_call(torch_dev, name):
    """One append call holding chunks of several sequences at once (3, 1, 0, 17 and 40
    tokens, starting inside and at block boundaries), twice in a row; the cache must equal
    the one-shot quantization of the final sequences."""
    stop = np.array([10, 64, 33, 95], np.int32)
    first = [3, 1, 0, 17]
    second = [40, 2, 31, 1]
    lens = stop + np.array(first) + np.array(second)
    w = W.workload(name, batch=len(lens))
    say("append mixed chunks", name, stop.tolist(), lens.tolist())
    built = harness.build(w, lens=lens, stop=stop)
    p = stop.copy()
    for chunk in (first, second):
        harness.append_ranges(built, [(b, int(p[b]), int(p[b]) + chunk[b]) for b in range(len(lens))])
        p += np.array(chunk, np.int32)
    if w["attn"] == 0:
        check_gqa_cache(built)
    else:
        check_mla_cache(built)


def test_append_prefill_large_batch_path(torch_dev):
    """One append call of > 65536 (token, head) rows takes the throughput kernel; it must
    give the same bytes as the latency kernel and the oracle."""
    w = W.workload("qwen3_4b", batch=1)
    lens = np.array([9000], np.int32)
    say("append large batch", lens.tolist())
    built = harness.build(w, lens=lens)
    check_gqa_cache(built)


@pytest.mark.parametrize("fmt", [0, 1])
def test_append_mla_latent_tiles(torch_dev, fmt):
    """Latent tiles (16 x 16 NVFP4 / 32 x 32 MXFP4) with their scale search, incremental
    appends that re-quantize the open tile row, both code layouts, the bf16 rope copy."""
    w = W.workload("mla", batch=2, fmt=fmt)
    lens = np.array([100, 48], np.int32)
    say("append mla fmt %d" % fmt, lens.tolist())
    built = harness.build(w, lens=lens, stop=np.array([60, 48]))
    harness.append_range(built, 0, 60, 61)
    harness.append_range(built, 0, 61, 100)
    check_mla_cache(built)


def test_decode_tiny_nvfp4(torch_dev):
    w = W.workload("tiny")
    say("decode tiny")
    built = harness.build(w)
    worst, worst_ref, zg, zo = compare_gqa(built, tol=TOL)
    say("tiny: max err vs oracle %.3g, vs fp64 attention %.3g, zero blocks gpu %d oracle %d"
        % (worst, worst_ref, zg, zo))


@pytest.mark.parametrize("hq", [64, 32, 16, 8])   # query heads per KV head 8, 4, 2, 1
def test_decode_nvfp4_ragged(torch_dev, hq):
    w = W.workload("qwen3_4b", batch=5, hq=hq)
    lens = np.array([1, 129, 1000, 2500, 0], np.int32)
    say("decode nvfp4 ragged hq=%d" % hq, lens.tolist())
    built = harness.build(w, lens=lens)
    worst, worst_ref, zg, zo = compare_gqa(built, tol=TOL)
    say("max err vs oracle %.3g, vs fp64 %.3g, zero blocks %d/%d" % (worst, worst_ref, zg, zo))


@pytest.mark.parametrize("hq", [32, 16, 8, 4])   # query heads per KV head 8, 4, 2, 1
def test_decode_mxfp4_ragged(torch_dev, hq):
    w = W.workload("qwen3_30b_a3b", batch=4, hq=hq)
    lens = np.array([33, 128, 777, 3000], np.int32)
    say("decode mxfp4 ragged hq=%d" % hq, lens.tolist())
    built = harness.build(w, lens=lens)
    worst, worst_ref, zg, zo = compare_gqa(built, tol=TOL)
    say("max err vs oracle %.3g, vs fp64 %.3g" % (worst, worst_ref))


@pytest.mark.parametrize("name", ["qwen3_4b", "qwen3_30b_a3b"])
def test_decode_shares_span_units(torch_dev, name):
    """Every wave takes an equal share of all tiles of the batch: with a few tiles per
    (sequence, KV head) unit, one share runs from inside one unit across whole units (and
    empty sequences) into the next, and long units are split over several waves."""
    lens = np.array([1, 0, 130, 600, 0, 0, 257, 64, 1000, 5, 0, 385], np.int32)
    w = W.workload(name, batch=len(lens))
    say("decode shares across units", name, lens.tolist())
    built = harness.build(w, lens=lens)
    worst, worst_ref, zg, zo = compare_gqa(built, tol=TOL)
    say("max err vs oracle %.3g, vs fp64 %.3g" % (worst, worst_ref))


@pytest.mark.parametrize("name", ["qwen3_4b", "qwen3_30b_a3b"])
def test_decode_batch_over_64(torch_dev, name):
    """More than 64 sequences: the partition lookup scans the lengths 64 sequences at a
    time (batches up to 64 take a single pass); sampled (sequence, KV head) pairs match the
    oracle, among them sequences past the first 64."""
    rng = np.random.default_rng(17)
    lens = rng.integers(1, 700, size=100).astype(np.int32)
    lens[rng.random(100) < 0.15] = 0
    w = W.workload(name, batch=len(lens))
    say("decode batch 100", name)
    built = harness.build(w, lens=lens)
    pairs = [(b, h) for b in (0, 5, 63, 64, 65, 80, 99) for h in (0, w["hkv"] - 1)]
    worst, worst_ref, zg, zo = compare_gqa(built, pairs=pairs, tol=TOL)
    say("batch 100: max err vs oracle %.3g, vs fp64 %.3g" % (worst, worst_ref))


@pytest.mark.parametrize("name", ["qwen3_4b", "qwen3_30b_a3b"])
def test_partition_reads_every_tile_once(torch_dev, name):
    """The decode kernel's partition and tile loads (run without arithmetic by
    fp4kv_cache_read) read every byte of the cache exactly once: with whole-tile sequences
    the xor of everything read equals the xor of the four cache arrays."""
    import torch
    from fp4_kv_cache_amd import lib as L
    lens = np.array([256, 0, 1280, 128, 640, 0, 2048, 384] * 9, np.int32)   # 72 sequences
    w = W.workload(name, batch=len(lens))
    say("partition coverage", name, len(lens))
    built = harness.build(w, lens=lens)
    maxp = built.bt.shape[1]
    n = L.fp4kv_cache_read_sink_words(built.cache.desc, w["batch"], w["hq"], maxp * w["page"])
    sink = torch.zeros(n, dtype=torch.int32, device=built.device)
    L.check(L.fp4kv_cache_read(built.cache.desc, w["batch"], w["hq"], built.bt.data_ptr(), maxp,
                               built.seq_lens.data_ptr(), sink.data_ptr(), n,
                               torch.cuda.current_stream().cuda_stream), "cache_read")
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    want = np.uint32(0)
    for name_ in ("k_codes", "k_scales", "v_codes", "v_scales"):
        want ^= np.bitwise_xor.reduce(getattr(built.cache, name_).cpu().numpy().view(np.uint32).ravel())
    assert got == want, (hex(int(got)), hex(int(want)))


@pytest.mark.parametrize("name,page", [("qwen3_4b", 32), ("qwen3_4b", 128), ("qwen3_4b", 256),
                                       ("qwen3_30b_a3b", 32), ("qwen3_30b_a3b", 128), ("qwen3_30b_a3b", 256)])
def test_page_sizes(torch_dev, name, page):
    """Every compiled page size: cache bytes bit-exact, decode within tolerance (a tile spans
    four pages at 32 tokens, one page at 128, half a page at 256)."""
    lens = np.array([1, 300, 0, 1100], np.int32)
    w = W.workload(name, batch=len(lens), page=page)
    say("page size %d %s" % (page, name), lens.tolist())
    built = harness.build(w, lens=lens)
    check_gqa_cache(built)
    worst, worst_ref, zg, zo = compare_gqa(built, tol=TOL)
    say("max err vs oracle %.3g, vs fp64 %.3g" % (worst, worst_ref))


@pytest.mark.parametrize("name,page", [("mla", 32), ("mla", 128), ("mla_mxfp4", 32), ("mla_mxfp4", 256)])
def test_mla_page_sizes(torch_dev, name, page):
    lens = np.array([40, 520], np.int32)
    w = W.workload(name, batch=len(lens), page=page)
    say("mla page size %d %s" % (page, name), lens.tolist())
    built = harness.build(w, lens=lens)
    check_mla_cache(built)
    worst, worst_ref, zg = compare_mla(built, tol=TOL)
    say("max err vs oracle %.3g, vs fp64 %.3g" % (worst, worst_ref))


@pytest.mark.parametrize("name", ["qwen3_4b", "qwen3_30b_a3b", "mla", "mla_mxfp4"])
def test_block_table_entries_past_the_pages_unused(torch_dev, name):
    """Block-table entries past a sequence's pages may hold anything (here ids outside the
    cache, negative and huge): the decode never uses them, and the output matches the
    oracle."""
    import torch
    lens = np.array([130, 1, 700, 64], np.int32)
    w = W.workload(name, batch=len(lens))
    say("block table garbage", name, lens.tolist())
    built = harness.build(w, lens=lens)
    bt = built.bt_np.copy()
    npg = -(-lens // w["page"])
    rng = np.random.default_rng(3)
    for b in range(len(lens)):
        tail = bt.shape[1] - npg[b]
        if tail > 0:
            bt[b, npg[b]:] = rng.choice([-7, 1 << 30, -(1 << 31), 12345678], size=tail)
    built.bt = torch.from_numpy(bt).to(built.device)
    if w["attn"] == 0:
        worst, worst_ref, zg, zo = compare_gqa(built, tol=TOL)
    else:
        worst, worst_ref, zg = compare_mla(built, tol=TOL)
    say("block table garbage: max err vs oracle %.3g" % worst)


@pytest.mark.parametrize("name", ["qwen3_30b_a3b", "mla", "mla_mxfp4"])
def test_fp32_inputs(torch_dev, name):
    """fp32 keys, values and queries (the other configurations feed bf16; the tiny one
    covers GQA NVFP4 in fp32): the append's and the decode's fp32 input paths."""
    lens = np.array([300, 129], np.int32)
    w = W.workload(name, batch=len(lens), dtype="fp32")
    say("fp32 inputs", name, lens.tolist())
    built = harness.build(w, lens=lens)
    if w["attn"] == 0:
        check_gqa_cache(built)
        worst, worst_ref, zg, zo = compare_gqa(built, tol=TOL)
    else:
        check_mla_cache(built)
        worst, worst_ref, zg = compare_mla(built, tol=TOL)
    say("fp32 inputs: max err vs oracle %.3g, vs fp64 %.3g" % (worst, worst_ref))


@pytest.mark.parametrize("name", ["qwen3_4b", "qwen3_30b_a3b", "mla", "mla_mxfp4"])
def test_decode_all_sequences_empty(torch_dev, name):
    """A batch whose sequence lengths are all zero: no wave or workgroup has tiles, and
    every output row is exactly zero (GQA: the merge writes the zeros; MLA: likewise)."""
    import torch
    lens = np.array([64, 200, 1], np.int32)
    w = W.workload(name, batch=len(lens))
    say("decode all empty", name)
    built = harness.build(w, lens=lens)
    built.seq_lens.zero_()
    q = built.queries()
    out = built.cache.decode(q, built.bt, built.seq_lens, W.softmax_scale(w))
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert o.shape[0] == len(lens) and not np.any(o), "non-zero output for empty sequences"


@pytest.mark.parametrize("name", ["mla", "mla_mxfp4"])
def test_decode_mla_many_splits(torch_dev, name):
    """One sequence with few head groups is split into more shares than the MLA merge loads
    at once (12 shares of 3-4 tiles for 6000 tokens and 16 heads), so the merge takes its
    general path; the output still matches the oracle."""
    lens = np.array([6000], np.int32)
    w = W.workload(name, batch=1, hq=16)
    say("decode %s many splits" % name, lens.tolist())
    built = harness.build(w, lens=lens)
    worst, worst_ref, zg = compare_mla(built, tol=TOL)
    say("mla many splits: max err vs oracle %.3g, vs fp64 attention %.3g" % (worst, worst_ref))


@pytest.mark.parametrize("name,hq", [("mla", 16), ("mla", 48), ("mla_mxfp4", 16), ("mla_mxfp4", 80)])
def test_decode_mla_head_counts(torch_dev, name, hq):
    """MLA workgroups serve four groups of 16 query heads; head counts that leave some of a
    workgroup's waves without a group (16 heads: three idle per role; 48 and 80: a partly
    filled quad) still stage tiles and join every barrier, and the active groups match the
    oracle."""
    lens = np.array([300, 1025], np.int32)
    w = W.workload(name, batch=len(lens), hq=hq)
    say("decode %s hq=%d" % (name, hq), lens.tolist())
    built = harness.build(w, lens=lens)
    worst, worst_ref, zg = compare_mla(built, tol=TOL)
    say("mla hq=%d: max err vs oracle %.3g, vs fp64 attention %.3g, zero blocks %d" % (hq, worst, worst_ref, zg))


@pytest.mark.parametrize("name,hq,n", [("qwen3_4b", 32, 2), ("qwen3_4b", 16, 4), ("qwen3_4b", 8, 8),
                                       ("qwen3_4b", 8, 3), ("qwen3_30b_a3b", 32, 2), ("qwen3_30b_a3b", 16, 4),
                                       ("qwen3_30b_a3b", 8, 7),
                                       # pages of 16, fp32 inputs; with 2 KV heads the partition
                                       # starts a share at the 129-token sequence's second tile,
                                       # which holds none of its first row's tokens
                                       ("tiny", 8, 2), ("tiny", 4, 4),
                                       # NVFP4 with 16 stacked query rows (two row sets of 8)
                                       ("qwen3_4b", 32, 4), ("qwen3_4b", 64, 2), ("tiny", 16, 2)])
def test_decode_multi_token(torch_dev, name, hq, n):
    """Several query tokens per sequence (causal), stacked on the same key / value tiles in
    one or two row sets; lengths put the shorter rows' last tile empty (129 = 128 + 1) and
    across a page boundary."""
    lens = np.array([n, 129, 0, 700, 1000 + n], np.int32)
    w = W.workload(name, batch=len(lens), hq=hq)
    say("decode multi-token %s hq=%d n=%d" % (name, hq, n), lens.tolist())
    built = harness.build(w, lens=lens)
    worst, worst_ref, zg, zo = compare_gqa_multi(built, n, tol=TOL)
    say("max err vs oracle %.3g, vs fp64 %.3g, zero blocks gpu %d oracle %d" % (worst, worst_ref, zg, zo))
    assert zg == zo


@pytest.mark.parametrize("name,hq,n,page", [("qwen3_4b", 32, 2, 32), ("qwen3_4b", 16, 3, 128),
                                            ("qwen3_4b", 8, 5, 256), ("qwen3_30b_a3b", 32, 2, 32),
                                            ("qwen3_30b_a3b", 16, 4, 128), ("qwen3_30b_a3b", 8, 6, 256)])
def test_decode_multi_token_page_sizes(torch_dev, name, hq, n, page):
    """Multi-token decode with pages of 32, 128 and 256 tokens (one, two or four 128-token
    tiles per page boundary case)."""
    lens = np.array([n, 129, 300, 700 + n], np.int32)
    w = W.workload(name, batch=len(lens), hq=hq, page=page)
    say("decode multi-token %s hq=%d n=%d page=%d" % (name, hq, n, page), lens.tolist())
    built = harness.build(w, lens=lens)
    worst, worst_ref, zg, zo = compare_gqa_multi(built, n, tol=TOL)
    say("max err vs oracle %.3g, vs fp64 %.3g" % (worst, worst_ref))
    assert zg == zo


def test_decode_underflow_no_zero_blocks(torch_dev):
    w = W.workload("long_underflow", batch=1)
    lens = np.array([16384], np.int32)
    say("decode underflow", lens.tolist())
    built = harness.build(w, lens=lens)
    worst, worst_ref, zg, zo = compare_gqa(built, pairs=[(0, 0), (0, 5)], tol=TOL)
    say("underflow: err %.3g, zero blocks gpu %d oracle %d" % (worst, zg, zo))
    assert zg == 0 and zo == 0


@pytest.mark.parametrize("name,hq", [("tiny", 8), ("qwen3_30b_a3b", 16), ("mla", 16), ("mla_mxfp4", 16)])
def test_special_values(torch_dev, name, hq):
    """Keys, values and the MLA latent with token rows of zeros, negative zeros, one constant,
    E2M1 grid values times powers of two (rounding ties) and single elements of 1000
    (``special_rows``): all-zero blocks (scale 0, signed zero codes), tie-breaking in the
    element rounding and the scale search, and large tensor scales.  The cache bytes equal the
    oracle's and the decode matches it.  The 1000-valued elements set the tensor scales, so the
    method's own error against fp64 attention is larger than on Gaussian data (the oracle's:
    0.42 for the NVFP4 GQA case, 0.25 MXFP4, 0.13 and 0.08 for the two latents); the bound
    against fp64 attention is 0.6 here."""
    w = W.workload(name, batch=2, hq=hq, degenerate=True)
    lens = np.array([300, 77], np.int32)
    say("special values %s hq=%d" % (name, hq), lens.tolist())
    built = harness.build(w, lens=lens)
    if w["attn"] == W.MLA:
        check_mla_cache(built)
        worst, worst_ref, zg = compare_mla(built, tol=TOL, ref_bound=0.6)
    else:
        check_gqa_cache(built)
        worst, worst_ref, zg, zo = compare_gqa(built, tol=TOL, ref_bound=0.6)
        assert zg == zo
    say("special values: max err vs oracle %.3g, vs fp64 attention %.3g" % (worst, worst_ref))


@pytest.mark.parametrize("name,hq", [("tiny", 8), ("qwen3_30b_a3b", 16), ("mla", 16), ("mla_mxfp4", 16)])
def test_scales_past_the_calibration(torch_dev, name, hq):
    """The special-value rows with the second sequence's keys, values and latent 2^20 times
    larger than the calibration sequence's: its NVFP4 block scales saturate at E4M3 448 (code
    0x7E, the search candidates clamped to [1, 0x7E]) and its FP4 codes at 6, while MXFP4 only
    shifts its E8M0 exponents.  Cache bytes equal the oracle's and the decode matches it; the
    saturation is deliberate, so the error against fp64 attention is not bounded here."""
    w = W.workload(name, batch=2, hq=hq, degenerate=True, seq_scales=(1.0, 2.0 ** 20))
    lens = np.array([300, 77], np.int32)
    say("scales past the calibration %s hq=%d" % (name, hq), lens.tolist())
    built = harness.build(w, lens=lens)
    if w["attn"] == W.MLA:
        check_mla_cache(built)
        worst, worst_ref, zg = compare_mla(built, tol=TOL, ref_bound=float("inf"))
    else:
        check_gqa_cache(built)
        worst, worst_ref, zg, zo = compare_gqa(built, tol=TOL, ref_bound=float("inf"))
        assert zg == zo
    say("scales past the calibration: max err vs oracle %.3g" % worst)


@pytest.mark.parametrize("name", ["mla", "mla_mxfp4"])
def test_decode_mla_ragged(torch_dev, name):
    """MLA: 128 query heads on one latent head (key and value) plus the bf16 rope part;
    NVFP4 (16 x 16 E4M3 tiles, FP4 matrix cores with signed-digit scale passes) and MXFP4
    (32 x 32 E8M0 tiles, FP4 matrix cores with the tile scales applied natively)."""
    w = W.workload(name, batch=4)
    lens = np.array([1, 200, 777, 0], np.int32)
    say("decode %s ragged" % name, lens.tolist())
    built = harness.build(w, lens=lens)
    worst, worst_ref, zg = compare_mla(built, tol=TOL)
    say("mla: max err vs oracle %.3g, vs fp64 attention %.3g, zero blocks %d" % (worst, worst_ref, zg))


@pytest.mark.parametrize("name,lens,hq,page", [
    # GQA NVFP4, 16-token pages: the window holds 64 tiles; one share of 71 tiles per unit
    ("tiny", [9000], 8, 16),
    # GQA MXFP4, 64-token pages: the window holds 256 tiles; one wave streams 4 units of 259 tiles
    ("qwen3_30b_a3b", [33100], 32, 64),
    # MLA, 32-token pages: the window holds 128 tiles; one share of 134 tiles (and a second sequence)
    ("mla", [17100, 300], 16, 32),
    ("mla_mxfp4", [17100, 300], 16, 32),
])
def test_decode_long_shares_restage_page_ids(torch_dev, name, lens, hq, page, monkeypatch):
    """With the decode limited to one share (FP4KV_MAX_SHARES=1) a share runs past the page-id
    window the kernels hold in LDS and re-stages it; the output still matches the oracle."""
    monkeypatch.setenv("FP4KV_MAX_SHARES", "1")
    lens = np.array(lens, np.int32)
    w = W.workload(name, batch=len(lens), hq=hq, page=page)
    say("decode long shares %s" % name, lens.tolist())
    built = harness.build(w, lens=lens)
    if w["attn"] == 0:
        pairs = [(0, h) for h in range(min(w["hkv"], 2))] + [(0, w["hkv"] - 1)]
        worst, worst_ref, zg, zo = compare_gqa(built, pairs=pairs, tol=TOL)
    else:
        worst, worst_ref, zg = compare_mla(built, tol=TOL)
    say("long shares: max err vs oracle %.3g, vs fp64 %.3g" % (worst, worst_ref))


@pytest.mark.parametrize("name", ["qwen3_4b", "mla"])
def test_workspace_from_a_bound_below_the_block_table(torch_dev, name):
    """The workspace size query takes any bound on the sequence lengths: a workspace sized for
    max(seq_lens) is accepted by a decode whose block table names far more pages."""
    import torch
    lens = np.array([130, 700], np.int32)
    w = W.workload(name, batch=len(lens))
    say("workspace bound", name, lens.tolist())
    built = harness.build(w, lens=lens)
    wide = np.zeros((len(lens), built.bt_np.shape[1] + 40), np.int32)
    wide[:, :built.bt_np.shape[1]] = built.bt_np
    built.bt_np = wide
    built.bt = torch.from_numpy(wide).to(built.device)
    q = built.queries()
    nb = built.cache.workspace_bytes(len(lens), w["hq"], int(lens.max()))
    ws = torch.empty(nb, dtype=torch.uint8, device=built.device)
    out = built.cache.decode(q, built.bt, built.seq_lens, W.softmax_scale(w), workspace=ws)
    ref = built.cache.decode(q, built.bt, built.seq_lens, W.softmax_scale(w))
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    if w["attn"] == 0:
        compare_gqa(built, tol=TOL)
    else:
        compare_mla(built, tol=TOL)


@pytest.mark.parametrize("name,dtype", [("mla", "bf16"), ("mla_mxfp4", "bf16"), ("mla", "fp32"),
                                        ("mla_mxfp4", "fp32")])
def test_mla_prepared_query_is_the_oracles(torch_dev, name, dtype):
    """The MLA query that the partial kernel consumes -- smoothed, rotated, dual-residual FP4 --
    read back from the workspace (the last batch * heads records of the reported size): the
    codes of both passes, the block scale bytes of valid blocks and the two tensor scales equal
    the oracle's quantize_query bit for bit, and the rope query is the input rounded to bf16.
    This is the query-code agreement measured directly, for every row of the batch."""
    import torch
    from oracle import query as QY
    lens = np.array([300, 0, 1025], np.int32)
    w = W.workload(name, batch=len(lens), hq=48, dtype=dtype)
    say("prepared query", name, dtype, lens.tolist())
    built = harness.build(w, lens=lens)
    q = built.queries()
    B, hq, D = len(lens), w["hq"], w["d"]
    nb = built.cache.workspace_bytes(B, hq, built.bt.shape[1] * w["page"])
    ws = torch.zeros(nb, dtype=torch.uint8, device=built.device)
    built.cache.decode(q, built.bt, built.seq_lens, W.softmax_scale(w), workspace=ws)
    torch.cuda.synchronize()
    rec = ws[nb - B * hq * 768:].cpu().numpy().reshape(B, hq, 768)
    qn = q.float().cpu().numpy()
    qs = built.calib[1][0]
    blk = 16 if w["fmt"] == W.NVFP4 else 32
    for b in range(B):
        qq = QY.quantize_query(qn[b, :, :D], qs, w["fmt"])
        for k, (c, e, v, G) in enumerate(((qq.c1, qq.e1, qq.v1, qq.G1), (qq.c2, qq.e2, qq.v2, qq.G2))):
            packed = rec[b, :, 256 * k:256 * (k + 1)]
            got = np.stack([packed & 0xF, packed >> 4], axis=-1).reshape(hq, D)
            bad = np.argwhere(got != c)
            assert bad.size == 0, "seq %d pass %d: %d code mismatches, first (head, channel) %s" % (
                b, k + 1, len(bad), bad[0].tolist())
            sb = rec[b, :, 512 + 32 * k:512 + 32 * k + D // blk].astype(np.int32)
            want = np.asarray(e, np.int32) + 127
            assert np.array_equal(np.where(v, sb, 0), np.where(v, want, 0)), (b, k)
            gs = rec[b, :, 576 + 4 * k:580 + 4 * k].copy().view(np.float32).ravel()
            assert np.array_equal(gs.view(np.uint32), np.asarray(G, np.float32).view(np.uint32)), (b, k)
        rope = rec[b, :, 640:768].copy().view(np.uint16)
        assert np.array_equal(rope, W.bf16_bits(W.bf16_round(qn[b, :, D:]))), b
    say("prepared query: %d rows, both passes bit-exact" % (B * hq))
