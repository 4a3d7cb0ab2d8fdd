"""Parity of the HIP path (through the C ABI) with the CPU oracle on seeded
inputs, element by element, per parameter tensor.

fp32 cases: loss relative error <= 1e-4 and per-tensor gradient relative
L2 error <= 1e-4 against the float64 oracle. bf16 cases: loss relative error
<= 1e-2 and per-tensor gradient cosine >= 0.999.

Shapes: the tiny configuration, plus variants that span several tiles of
every kernel and end in ragged tails (sequence lengths that are not a
multiple of any tile, GQA, head_dim 128, ignored targets, accumulation).
"""
import numpy as np
import pytest

import oracle
import workloads as W
from decoder_only_pretraining_amd import binding as B
from tests.gpu_common import (assert_bf16_parity, assert_fp32_parity, gpu_step, inputs,
                              per_tensor)

pytestmark = pytest.mark.gpu

TINY = W.get("tiny")
CASES = {
    "tiny": TINY,
    # 4 layers (SSSL), GQA 4:2, ragged T and B, window edge inside tiles
    "ragged_gqa": TINY.with_(name="ragged_gqa", n_layer=4, n_head=4, n_kv_head=2, seq_len=77,
                             batch=3, short_window=20, vocab=448, mlp_hidden=320),
    # head_dim 128, 3 layers (ve on 0 and 2), T spans two query tiles
    "d128": TINY.with_(name="d128", n_layer=3, n_embd=256, n_head=2, n_kv_head=1, head_dim=128,
                       mlp_hidden=512, seq_len=150, batch=2, short_window=37, vocab=640),
    # one token per row
    "t1": TINY.with_(name="t1", seq_len=1, batch=5, short_window=0),
}


@pytest.mark.parametrize("name", list(CASES))
def test_fp32_parity(name):
    w = CASES[name]
    p, tok, tgt = inputs(w, wseed=100 + len(name), tseed=200 + len(name))
    lo, go = oracle.forward_backward(w, p.astype(np.float64), tok, tgt)
    lg, gg, _ = gpu_step(w, p, tok, tgt)
    # with one key per query, attention returns v and q, k get no gradient
    zero = [f"l{l}.{x}" for l in range(w.n_layer) for x in "qk"] if w.seq_len == 1 else []
    assert_fp32_parity(w, lg, gg, lo, go, zero=zero)


def test_ignored_targets_and_accumulate():
    import torch
    w = CASES["ragged_gqa"]
    p, tok, tgt = inputs(w, 5, 6)
    tgt = tgt.copy()
    tgt[0, :30] = -1
    tgt[2, 50:] = -1
    lo, go = oracle.forward_backward(w, p.astype(np.float64), tok, tgt)
    step = B.Step(w, p, tok, tgt, flags=B.GPT_F_ACCUMULATE)
    # the buffer starts at the oracle's gradient (same scale per tensor, so
    # the difference below loses no precision); two calls then add 2 g
    prior = go.astype(np.float32)
    step.grads.copy_(torch.from_numpy(prior))
    step.run()
    step.run()
    torch.cuda.synchronize()
    g = (step.grads.cpu().numpy().astype(np.float64) - prior) / 2
    assert_fp32_parity(w, float(step.loss.item()), g, lo, go)


def test_all_targets_ignored_gives_zero():
    import torch
    w = TINY
    p, tok, tgt = inputs(w, 8, 9)
    tgt = np.full_like(tgt, -1)
    lg, gg, _ = gpu_step(w, p, tok, tgt)
    assert lg == 0.0
    assert np.all(gg == 0.0)


def test_zero_lm_head_loss_is_ln_vocab():
    w = TINY
    p, tok, tgt = inputs(w)
    o, s = oracle.param_offsets(w)[0]["lm_head"]
    p[o:o + s[0] * s[1]] = 0
    lg, _, _ = gpu_step(w, p, tok, tgt)
    assert abs(lg - np.log(w.vocab)) < 1e-5


def test_repeatable():
    """Two calls on the same inputs agree; only the atomics-accumulated
    embedding gradients may differ by rounding order."""
    import torch
    w = CASES["ragged_gqa"]
    p, tok, tgt = inputs(w)
    step = B.Step(w, p, tok, tgt)
    step.run()
    torch.cuda.synchronize()
    l1, g1 = step.loss.item(), step.grads.cpu().numpy().copy()
    step.run()
    torch.cuda.synchronize()
    l2, g2 = step.loss.item(), step.grads.cpu().numpy()
    assert l1 == l2
    for name, (rel, cos) in per_tensor(w, g2, g1).items():
        assert rel <= 1e-6, name


def test_reused_weight_mirrors_give_the_same_step():
    """GPT_F_REUSE_WEIGHTS on the call after one with the same params and
    workspace: the bf16 mirrors left by the first call are what a fresh
    conversion would write, so loss and gradients are bit-identical."""
    import torch
    w = SMALL_BF16
    p, tok, tgt = inputs(w, 33, 34)
    step = B.Step(w, p, tok, tgt)
    step.run()
    torch.cuda.synchronize()
    l1, g1 = step.loss.item(), step.grads.cpu().numpy().copy()
    cfg = B.make_config(w, B.GPT_F_REUSE_WEIGHTS)
    B.fwd_bwd(cfg, step.params, step.tokens, step.targets, step.loss, step.grads, step.workspace)
    torch.cuda.synchronize()
    assert step.loss.item() == l1
    g2 = step.grads.cpu().numpy()
    offs = oracle.param_offsets(w)[0]
    for name, (o, s) in offs.items():   # tables take fp32 atomics: order-dependent sums
        n = int(np.prod(s))
        if name == "wte" or name.endswith(".ve"):
            assert per_tensor(w, g2, g1)[name][0] <= 1e-6, name
        else:
            assert np.array_equal(g2[o:o + n], g1[o:o + n]), name


SMALL_BF16 = W.get("d12").with_(name="small_bf16", n_layer=4, seq_len=300, batch=2,
                                short_window=75, vocab=2048)
SMALL_BF16_GQA = SMALL_BF16.with_(name="small_bf16_gqa", n_kv_head=2, seq_len=256, batch=3,
                                  short_window=64)


# d26 widths in bf16: 13 KV heads x 1664 fp32 gate weights (86.5 KB) take
# the mix/norm kernel's 1024-thread path, which stages them in one LDS copy
# per CU; layer 1 (the last) carries value embeddings.
SMALL_D26W = W.get("d26").with_(name="small_d26w", n_layer=2, seq_len=200, batch=2,
                                short_window=50, vocab=2048, fp8_linears=False)


@pytest.mark.parametrize("w", [SMALL_BF16, SMALL_BF16_GQA, SMALL_D26W], ids=lambda w: w.name)
def test_bf16_parity_small(w):
    """The bf16 kernels at d12 widths (C 768, D 128, F 3072) and d26 widths
    (C 1664, 13 heads, F 6656) on a short sequence, against the float64
    oracle."""
    p, tok, tgt = inputs(w, 31, 32)
    lo, go = oracle.forward_backward(w, p.astype(np.float64), tok, tgt)
    lg, gg, _ = gpu_step(w, p, tok, tgt)
    assert_bf16_parity(w, lg, gg, lo, go)


# 16,384 tokens at d12 widths: the same tile shapes and K splits the full d12
# step takes (256x256 and 256x192 output tiles, split-K weight gradients and
# vocabulary-split logit gradient), against the float64 oracle.
MID_BF16 = W.get("d12").with_(name="mid_bf16", n_layer=2, seq_len=256, batch=64,
                              short_window=64, vocab=8192)


def test_bf16_parity_mid():
    w = MID_BF16
    p, tok, tgt = inputs(w, 41, 42)
    lo, go = oracle.forward_backward(w, p.astype(np.float64), tok, tgt)
    lg, gg, _ = gpu_step(w, p, tok, tgt)
    assert_bf16_parity(w, lg, gg, lo, go)
