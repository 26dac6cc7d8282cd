"""Per-technique ablation on the GPU: the ablation-study build of the library
(libfp4kv_ablate.so, the same sources with -DFP4KV_ABLATION) switches one technique of the
method off at a time -- the dual-residual query, the Hadamard rotation, the key scale search;
static smoothing is switched off through its inputs (all-ones smoothing vectors) -- and must
match the oracle with the same switch: cache bytes bit-exact, decode rows within 1e-3 of the
row norm.  The error against unquantized fp64 attention is printed for each setting (the GPU
rows of the ablation table).  The product library contains none of the switches."""
import numpy as np
import pytest

from fp4_kv_cache_amd import workloads as W
from fp4_kv_cache_amd import harness
from _gpu import say, check_gqa_cache, compare_gqa

pytestmark = pytest.mark.gpu
TOL = 1e-3


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "GPU test run without a GPU"
    from fp4_kv_cache_amd import lib
    lib.load()
    lib.load_ablation()
    return torch


SETTINGS = [
    ("full method", 0, {}),
    ("single-pass query (no dual residual)", 1, {"dual": False}),
    ("no Hadamard rotation", 2, {"rotate": False}),
    ("no key scale search", 4, {"search": False}),
    ("no smoothing", 0, {"smooth": False}),
]


@pytest.mark.parametrize("name", ["qwen3_4b", "qwen3_30b_a3b"])
@pytest.mark.parametrize("label,flags,opts", SETTINGS, ids=[s[0].split(" (")[0] for s in SETTINGS])
def test_ablation_switch_matches_oracle(torch_dev, name, label, flags, opts):
    from fp4_kv_cache_amd import lib as L
    lens = np.array([700, 129, 2100], np.int32)
    w = W.workload(name, batch=len(lens))
    calib = None
    if not opts.get("smooth", True):
        ksi, qs, gk, gv = W.calibration(w)
        calib = (np.ones_like(ksi), np.ones_like(qs), gk, gv)
    say("ablation %s: %s" % (name, label), lens.tolist())
    with L.ablation(flags):
        built = harness.build(w, lens=lens, calib=calib)
        check_gqa_cache(built, opts=opts)
        worst, worst_ref, zg, zo = compare_gqa(built, tol=TOL, opts=opts, ref_bound=1.5)
    say("ABLATION %s | %s | max err vs oracle %.3g | error vs fp64 attention over all rows %.4f"
        % (name, label, worst, compare_gqa.last_agg))
