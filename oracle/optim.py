"""MuonAdamW optimizer step (test infrastructure only).

What the pages fix ("NanoChat基础训练报告", optimizer block; "Nanochat在nanoGPT
之上的新增功能", feature table row on the optimizer and the notes on Muon;
"nanochat — 架构与原理", section 3 on MuonAdamW):
  * matrix parameters take Muon: momentum, then Newton-Schulz
    orthogonalisation of the update; embeddings and scalars take AdamW;
  * learning rates: matrices 0.02, scalars 0.5, embeddings 0.3, the
    unembedding (lm_head) 0.008; weight decay 0.28; the schedule (40 warmup
    steps, decay from 65% of training to 0.05) is a multiplier the caller
    applies to every rate.
Readings where the pages are silent (each an input of the step, so a
caller can set it; the defaults follow the published Muon and AdamW
descriptions): Muon momentum 0.95 with the Nesterov form, the quintic
Newton-Schulz iteration X <- a X + (b A + c A^2) X, A = X X^T, on the
update scaled to unit Frobenius norm (taken on the wide orientation, rows
<= cols), coefficients (3.4445, -4.7750, 2.0315), 5 steps, the result
scaled by sqrt(max(1, rows / cols)); AdamW betas (0.9, 0.999), eps 1e-8,
bias-corrected; the weight decay applies (decoupled, times the rate) to the
Muon matrices only. Groups: Muon for the six block linears of every layer;
AdamW with the embedding rate for wte and the value-embedding tables, the
unembedding rate for lm_head, the scalar rate for the lambdas, the
value-embedding gates and the Smear / Backout parameters.
"parity unpinned" with respect to the pages for the readings above; the
arithmetic is pinned in the tests (torch's AdamW, the polar factor from an
SVD, closed forms).
"""
from __future__ import annotations

import numpy as np

from .model import param_offsets, unpack

DEFAULTS = dict(lr_matrix=0.02, lr_scalar=0.5, lr_embed=0.3, lr_unembed=0.008,
                weight_decay=0.28, lr_mult=1.0, beta1=0.9, beta2=0.999, eps=1e-8,
                momentum=0.95, nesterov=True, ns_a=3.4445, ns_b=-4.7750, ns_c=2.0315,
                ns_steps=5)


def adamw_update(p, g, m, v, lr, t, beta1, beta2, eps, wd=0.0):
    """One AdamW step on arrays in place (t = 1, 2, ...): moments, bias
    correction, decoupled decay p *= 1 - lr wd."""
    m *= beta1
    m += (1 - beta1) * g
    v *= beta2
    v += (1 - beta2) * g * g
    mh = m / (1 - beta1 ** t)
    vh = v / (1 - beta2 ** t)
    p *= 1 - lr * wd
    p -= lr * mh / (np.sqrt(vh) + eps)


def newton_schulz(G, a, b, c, steps, eps=1e-7):
    """Approximate orthogonalisation of G: X = G / (||G||_F + eps) in the
    orientation with rows <= cols, then `steps` times X <- a X + (b A + c A^2) X
    with A = X X^T; returned in G's orientation."""
    X = np.asarray(G, dtype=np.float64) / (np.linalg.norm(G) + eps)
    wide = X.shape[0] <= X.shape[1]
    if not wide:
        X = X.T
    for _ in range(steps):
        A = X @ X.T
        X = a * X + (b * A + c * (A @ A)) @ X
    return X if wide else X.T


def muon_update(p, g, buf, lr, momentum, nesterov, wd, a, b, c, steps):
    """One Muon step on a [rows, cols] matrix in place: buf <- mu buf + g;
    u = g + mu buf (Nesterov) or buf; p <- p (1 - lr wd) - lr sqrt(max(1,
    rows / cols)) NS(u)."""
    buf *= momentum
    buf += g
    u = g + momentum * buf if nesterov else buf
    O = newton_schulz(u, a, b, c, steps)
    scale = max(1.0, p.shape[0] / p.shape[1]) ** 0.5
    p *= 1 - lr * wd
    p -= lr * scale * O


def group(name: str):
    """(rule, learning-rate key) of a parameter tensor."""
    leaf = name.split(".")[-1]
    if leaf in ("q", "k", "v", "o", "fc", "mp"):
        return "muon", "lr_matrix"
    if name == "wte" or leaf == "ve":
        return "adamw", "lr_embed"
    if name == "lm_head":
        return "adamw", "lr_unembed"
    return "adamw", "lr_scalar"   # lambdas, value-embedding gates, smear gate, backout lambda


def optimizer_step(cfg, params, grads, m, v, step, **hp):
    """One MuonAdamW step over the flat fp64 arrays in place. m: AdamW first
    moment / Muon momentum buffer; v: AdamW second moment (unused by Muon
    tensors). step: 1, 2, ... (AdamW bias correction)."""
    h = dict(DEFAULTS, **hp)
    P, G, M, Vv = (unpack(cfg, x) for x in (params, grads, m, v))
    for name in param_offsets(cfg)[0]:
        rule, key = group(name)
        lr = h[key] * h["lr_mult"]
        if rule == "muon":
            muon_update(P[name], G[name], M[name], lr, h["momentum"], h["nesterov"],
                        h["weight_decay"], h["ns_a"], h["ns_b"], h["ns_c"], h["ns_steps"])
        else:
            adamw_update(P[name], G[name], M[name], Vv[name], lr, step, h["beta1"], h["beta2"],
                         h["eps"])
