"""The fp8 parity bar (tests/gpu_common.fp8_bounds) is not vacuous: a
mistake planted in the oracle, on the CPU, fails it, while the oracle's own
bf16-rounding variant passes it."""
import numpy as np

import oracle
import workloads as W
from oracle import model as M
from tests.gpu_common import fp8_bounds, per_tensor

CFG = W.get("d12").with_(name="fp8_bar", n_layer=2, n_embd=256, n_head=2, n_kv_head=1,
                         mlp_hidden=1024, vocab=512, seq_len=96, batch=2, short_window=24,
                         fp8_linears=True)


def _run(lin_cls=None, **kw):
    _, total = oracle.param_offsets(CFG)
    p = W.gen_params(total, CFG.n_layer, 61)
    tok, tgt = W.split_tokens(W.gen_tokens(CFG, 62))
    orig = M._Lin
    if lin_cls is not None:
        M._Lin = lin_cls
    try:
        return oracle.forward_backward(CFG, p, tok, tgt, dtype=np.float32, **kw)
    finally:
        M._Lin = orig


class _WrongBackwardScale(M._Lin):
    """Planted mistake: the weight operand of the backward products
    dequantised with a scale 25% off."""

    def bwd(self, gy, x, W):
        gx, gw = super().bwd(gy, x, W)
        return gx * np.float32(1.25), gw


def _failures(grads, go, gr):
    spread = {k: v[0] for k, v in per_tensor(CFG, gr, go).items()}
    bound = fp8_bounds(CFG, spread)
    return {k for k, v in per_tensor(CFG, grads, go).items() if not v[0] <= bound[k]}


def test_fp8_bar_accepts_variant_and_rejects_planted_mistake():
    _, go = _run()
    _, gr = _run(fp8_round="bf16")
    _, gm = _run(_WrongBackwardScale)
    assert not _failures(gr, go, gr)
    bad = _failures(gm, go, gr)
    # every tensor upstream of the first backward product moves by ~25%
    assert len(bad) >= len(oracle.param_offsets(CFG)[0]) // 2, bad
