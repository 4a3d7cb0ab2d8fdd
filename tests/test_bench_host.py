"""The benchmark's own size and FLOP accounting agrees with the oracle's
parameter layout and model-FLOP count (no GPU)."""
import pytest

import bench
import oracle
import workloads as W

CASES = [W.get(n) for n in W.CONFIGS] + [
    W.get("d12").with_(smear=True), W.get("d12").with_(backout=True),
    W.get("tiny").with_(smear=True, backout=True)]


@pytest.mark.parametrize("w", CASES, ids=lambda w: f"{w.name}-{int(w.smear)}{int(w.backout)}")
def test_param_total_and_flops_match_oracle(w):
    assert bench.param_total(w) == oracle.param_offsets(w)[1]
    assert bench.model_flops_per_token(w) == pytest.approx(oracle.model_flops_per_token(w),
                                                           rel=1e-12)


# Model MFLOP per token (fwd + bwd: 6 per matrix weight used in a product
# plus 12 H D per visible key per layer) as worked out by hand from the five
# workload descriptions when the benchmark was planned; the d12 figure gives
# 11.900 TFLOP per 16,384-token call.
HAND = {"tiny": 2.83, "d12": 726.33, "d12_gqa": 669.59, "d20": 2793.82, "d26": 5825.72}


@pytest.mark.parametrize("name", list(HAND))
def test_model_flops_match_the_hand_count(name):
    assert bench.model_flops_per_token(W.get(name)) / 1e6 == pytest.approx(HAND[name], abs=0.006)
