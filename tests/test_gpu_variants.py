"""Parity of the Smear and Backout model variants (GPT_F_SMEAR,
GPT_F_BACKOUT) of the HIP path with the CPU oracle, at the bars of the
base model: fp32 loss and per-tensor gradient relative error <= 1e-4
against the float64 oracle; bf16 loss relative error <= 1e-2 and per-tensor
gradient cosine >= 0.999.

The smear gate is drawn 50x wider than the other weights so that the gates
spread over (0, 1) instead of sitting at 1/2, and the backout lambda is
0.5. Shapes cover the cached layer in the middle of the stack (3 layers:
layer 1), at layer 0 (1 layer: the stream cached is the embedding itself),
one token per sequence (no position has a predecessor), ragged lengths and
GQA, gradient accumulation, and d12 widths in bf16.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from decoder_only_pretraining_amd import binding as B
from tests.gpu_common import assert_bf16_parity, assert_fp32_parity, gpu_step, inputs

pytestmark = pytest.mark.gpu

TINY = W.get("tiny").with_(smear=True, backout=True)
CASES = {
    "tiny": TINY,
    "ragged_gqa_l3": TINY.with_(name="ragged_gqa_l3", n_layer=3, n_head=4, n_kv_head=2,
                                seq_len=77, batch=3, short_window=20, vocab=448,
                                mlp_hidden=320),
    "one_layer": TINY.with_(name="one_layer", n_layer=1, seq_len=40, batch=3),
    "t1": TINY.with_(name="t1", seq_len=1, batch=5, short_window=0),
    "smear_only": W.get("tiny").with_(name="smear_only", smear=True, n_layer=3, seq_len=50),
    "backout_only": W.get("tiny").with_(name="backout_only", backout=True, n_layer=4,
                                        seq_len=50),
}


def variant_inputs(w, wseed, tseed):
    p, tok, tgt = inputs(w, wseed, tseed)
    offs = oracle.param_offsets(w)[0]
    if w.smear:
        o = offs["smear_gate"][0]
        p[o:o + w.n_embd] *= 50
    if w.backout:
        p[offs["backout_lambda"][0]] = 0.5
    return p, tok, tgt


@pytest.mark.parametrize("name", list(CASES))
def test_fp32_parity_variants(name):
    w = CASES[name]
    p, tok, tgt = variant_inputs(w, 300 + len(name), 400 + len(name))
    lo, go = oracle.forward_backward(w, p.astype(np.float64), tok, tgt)
    lg, gg, _ = gpu_step(w, p, tok, tgt)
    zero = [f"l{l}.{x}" for l in range(w.n_layer) for x in "qk"] if w.seq_len == 1 else []
    if w.seq_len == 1 and w.smear:
        zero.append("smear_gate")     # no position has a predecessor
    assert_fp32_parity(w, lg, gg, lo, go, zero=zero)


def test_variants_accumulate():
    import torch
    w = CASES["ragged_gqa_l3"]
    p, tok, tgt = variant_inputs(w, 7, 8)
    lo, go = oracle.forward_backward(w, p.astype(np.float64), tok, tgt)
    step = B.Step(w, p, tok, tgt, flags=B.GPT_F_ACCUMULATE)
    prior = go.astype(np.float32)
    step.grads.copy_(torch.from_numpy(prior))
    step.run()
    step.run()
    torch.cuda.synchronize()
    g = (step.grads.cpu().numpy().astype(np.float64) - prior) / 2
    assert_fp32_parity(w, float(step.loss.item()), g, lo, go)


def test_forward_only_loss_matches():
    import torch
    w = CASES["ragged_gqa_l3"]
    p, tok, tgt = variant_inputs(w, 9, 10)
    lo = oracle.forward_loss(w, p.astype(np.float64), tok, tgt)
    step = B.Step(w, p, tok, tgt)
    step.forward()
    torch.cuda.synchronize()
    assert abs(float(step.loss.item()) - lo) <= 1e-4 * abs(lo)


SMALL_BF16 = W.get("d12").with_(name="small_bf16_sb", n_layer=4, seq_len=300, batch=2,
                                short_window=75, vocab=2048, smear=True, backout=True)


def test_bf16_parity_variants():
    """d12 widths (C 768, D 128, F 3072), 4 layers (the cached stream enters
    layer 2), bf16 compute, against the float64 oracle."""
    w = SMALL_BF16
    p, tok, tgt = variant_inputs(w, 51, 52)
    lo, go = oracle.forward_backward(w, p.astype(np.float64), tok, tgt)
    lg, gg, _ = gpu_step(w, p, tok, tgt)
    assert_bf16_parity(w, lg, gg, lo, go)
