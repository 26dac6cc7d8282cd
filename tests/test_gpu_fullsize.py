"""GPU parity at the workloads' full sizes, in the launch configuration bench.py times.

The whole batch is prefilled and decoded through the C ABI; the oracle then checks sampled
(sequence, KV head) units one at a time: cache codes and scales bit-exact, decode rows
within 1e-3 of the row norm.  The long-context stress workload also checks, over the
whole batch, that no probability block quantizes to all zeros.
"""
import numpy as np
import pytest

from fp4_kv_cache_amd import workloads as W
from fp4_kv_cache_amd import harness
from _gpu import say, check_gqa_cache, check_mla_cache, compare_gqa, compare_mla

pytestmark = pytest.mark.gpu
TOL = 1e-3


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "GPU test run without a GPU"
    from fp4_kv_cache_amd import lib
    lib.load()
    return torch


def _run(name, pairs):
    w = W.workload(name)
    say("full size %s: batch %d, hq %d, hkv %d, fmt %d; building cache" % (name, w["batch"], w["hq"], w["hkv"],
                                                                         w["fmt"]))
    built = harness.build(w, workers=16)
    say("  cache built, %d tokens in total; checking cache bytes of %s" % (int(built.lens.sum()), pairs))
    check_gqa_cache(built, pairs=pairs)
    say("  decoding the whole batch; checking %s" % (pairs,))
    worst, worst_ref, zg, zo = compare_gqa(built, pairs=pairs, tol=TOL)
    say("  max err vs oracle %.3g, vs fp64 attention %.3g, zero P blocks: gpu (whole batch) %d, oracle "
        "(sampled) %d" % (worst, worst_ref, zg, zo))
    return zg, zo


def test_fullsize_qwen3_4b_nvfp4(torch_dev):
    _run("qwen3_4b", [(0, 0), (7, 3), (15, 7)])


def test_fullsize_qwen3_30b_a3b_mxfp4(torch_dev):
    w = W.workload("qwen3_30b_a3b")
    lens = W.seq_lens(w)
    longest, shortest = int(np.argmax(lens)), int(np.argmin(lens))
    _run("qwen3_30b_a3b", [(longest, 0), (shortest, 3), (17, 2)])


def test_fullsize_long_underflow_no_zero_blocks(torch_dev):
    zg, zo = _run("long_underflow", [(0, 0), (3, 7)])
    assert zg == 0 and zo == 0


@pytest.mark.parametrize("name", ["mla", "mla_mxfp4"])
def test_fullsize_mla(torch_dev, name):
    w = W.workload(name)
    say("full size %s: batch %d, latent 512 + rope 64; building cache" % (name, w["batch"]))
    built = harness.build(w, workers=16)
    say("  checking latent codes, tile scales and rope of sequences 0 and 31")
    check_mla_cache(built, seqs=[0, 31])
    say("  decoding the whole batch; checking sequences 0 and 31")
    worst, worst_ref, zg = compare_mla(built, seqs=[0, 31], tol=TOL)
    say("  max err vs oracle %.3g, vs fp64 attention %.3g, zero P blocks (whole batch) %d" % (worst, worst_ref, zg))
