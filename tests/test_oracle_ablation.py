"""The oracle's technique switches move the error the way the method says they should.

The full study (tests/ablation.py) tabulates every switch on the five workloads; these
checks pin the effects that must hold by construction or by a wide margin:
* the key scale search never raises a block's reconstruction error (the default scale is
  the first candidate and only a strictly smaller objective replaces it),
* the dual-residual query lowers the logit error ("BitDecoding-FP4: Native FP4 KV Cache
  Decoding via Algorithm-System Co-Design", Article Summary),
* the tile-relative P with its 2^-10 tensor scale keeps every long-context probability
  block alive, while normalized P with tensor scale 1 loses them ("FP4 KV Cache Done Right",
  What is actually new in BitDecoding-FP4? -- Underflow-Aware Probability Scaling).
"""
import os
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import ablation  # noqa: E402


@pytest.mark.parametrize("name", ["qwen3_4b", "qwen3_30b_a3b"])
def test_search_never_raises_key_error(name):
    assert ablation.key_sse(name, 512, True) <= ablation.key_sse(name, 512, False)


def test_dual_residual_lowers_logit_error():
    plan = ([(0, 0), (3, 5)], 1024)
    full = ablation.run_setting("qwen3_4b", plan, {})
    single = ablation.run_setting("qwen3_4b", plan, {"dual": False})
    assert full[0] < 0.8 * single[0]


def test_underflow_aware_scaling_keeps_blocks():
    plan = ([(0, 0)], 8192)
    full = ablation.run_setting("long_underflow", plan, {})
    vanilla = ablation.run_setting("long_underflow", plan, {"p_mode": "vanilla"})
    assert full[3] == 0.0
    assert vanilla[3] > 0.99
    assert full[1] < 0.5 * vanilla[1]
