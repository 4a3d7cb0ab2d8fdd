"""Pins of the CPU oracle against things other than itself.

Each test checks the oracle against a value the pages print, a closed form,
an invariant, a library routine (torch CPU in float64), brute force on tiny
inputs, or finite differences. None of these tests touches the GPU library.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads as W

torch.set_grad_enabled(True)


def _tiny(**kw):
    return W.get("tiny").with_(**kw)


# ---------------------------------------------------------------- layout

def test_param_counts_match_report():
    """The d12 report prints 286.3M parameters, 261.1M of them non-embedding."""
    cfg = W.get("d12")
    offs, total = oracle.param_offsets(cfg)
    non_emb = total - np.prod(offs["wte"][1])
    assert round(total / 1e6, 1) == 286.3
    assert round(non_emb / 1e6, 1) == 261.1
    assert total == 286_288_920 and non_emb == 261_123_096


def test_param_counts_other_configs():
    got = {n: oracle.param_offsets(W.get(n))[1] for n in W.CONFIGS}
    assert got == {"tiny": 590_084, "d12": 286_288_920, "d12_gqa": 176_170_008,
                   "d20": 896_660_520, "d26": 1_682_066_100}


def test_every_tensor_is_64_aligned():
    for cfg in W.CONFIGS.values():
        offs, _ = oracle.param_offsets(cfg)
        for name, (o, s) in offs.items():
            if not name.endswith("lambdas"):
                assert o % 64 == 0, (cfg.name, name)


def test_layer_patterns():
    def pat(cfg):
        L = cfg.n_layer
        return ("".join("L" if oracle.layer_is_full(l, L) else "S" for l in range(L)),
                [l for l in range(L) if oracle.layer_has_ve(l, L)])
    assert pat(W.get("tiny")) == ("SL", [1])
    # the report: value embeddings on layers 1, 3, 5, 7, 9, 11 of d12
    assert pat(W.get("d12")) == ("SSSL" * 3, [1, 3, 5, 7, 9, 11])
    assert pat(W.get("d20")) == ("SSSL" * 5, list(range(1, 20, 2)))
    s26, ve26 = pat(W.get("d26"))
    assert s26 == "SSSL" * 6 + "SL" and s26[-1] == "L"      # last layer forced full
    assert ve26 == list(range(1, 26, 2)) and 25 in ve26


# ---------------------------------------------------------------- RMSNorm

def test_rms_matches_torch():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((7, 33)) * 3
    y, r = oracle.rms_fwd(x, 2.0 ** -23)
    ref = F.rms_norm(torch.from_numpy(x), (33,), eps=2.0 ** -23).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-14, atol=1e-14)
    # invariant: mean(y^2) = ms / (ms + eps)
    ms = np.mean(x * x, axis=-1)
    np.testing.assert_allclose(np.mean(y * y, axis=-1), ms / (ms + 2.0 ** -23), rtol=1e-13)


def test_rms_bwd_matches_autograd():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 16))
    gy = rng.standard_normal((5, 16))
    y, r = oracle.rms_fwd(x, 1e-5)
    xt = torch.from_numpy(x).requires_grad_()
    F.rms_norm(xt, (16,), eps=1e-5).backward(torch.from_numpy(gy))
    np.testing.assert_allclose(oracle.rms_bwd(gy, y, r), xt.grad.numpy(), rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- RoPE

def test_rope_invariants():
    rng = np.random.default_rng(2)
    T, D = 40, 64
    cos, sin = oracle.rope_tables(T, D, 10000.0)
    x = rng.standard_normal((1, T, 3, D))
    y = oracle.rope_fwd(x, cos, sin)
    # rotation: every (i, i + D/2) pair keeps its length
    h = D // 2
    np.testing.assert_allclose(x[..., :h] ** 2 + x[..., h:] ** 2,
                               y[..., :h] ** 2 + y[..., h:] ** 2, rtol=1e-12)
    # position 0 is the identity
    np.testing.assert_allclose(y[:, 0], x[:, 0], rtol=0, atol=0)
    # backward = inverse rotation
    np.testing.assert_allclose(oracle.rope_bwd(y, cos, sin), x, atol=1e-12)
    # <rope_m q, rope_n k> depends only on m - n
    q = np.broadcast_to(rng.standard_normal(D), (1, T, 1, D))
    k = np.broadcast_to(rng.standard_normal(D), (1, T, 1, D))
    qr, kr = oracle.rope_fwd(q, cos, sin), oracle.rope_fwd(k, cos, sin)
    d1 = np.dot(qr[0, 10, 0], kr[0, 3, 0])
    d2 = np.dot(qr[0, 30, 0], kr[0, 23, 0])
    assert abs(d1 - d2) < 1e-10
    # frequencies: pair i advances by theta^(-2i/D) per position
    assert abs(math.atan2(sin[1, 1], cos[1, 1]) - 10000.0 ** (-2 / D)) < 1e-14


def test_rope_then_norm_commutes():
    rng = np.random.default_rng(3)
    T, D = 9, 64
    cos, sin = oracle.rope_tables(T, D, 10000.0)
    x = rng.standard_normal((2, T, 2, D))
    a, _ = oracle.rms_fwd(oracle.rope_fwd(x, cos, sin), 2.0 ** -23)
    b = oracle.rope_fwd(oracle.rms_fwd(x, 2.0 ** -23)[0], cos, sin)
    np.testing.assert_allclose(a, b, atol=1e-13)


# ---------------------------------------------------------------- attention

def _loop_attention(q, k, v, full, Wn):
    """Brute force with scalar loops over (t, s)."""
    B, T, H, D = q.shape
    Hk = k.shape[2]
    G = H // Hk
    y = np.zeros_like(q)
    for b in range(B):
        for h in range(H):
            j = h // G
            for t in range(T):
                keys = [s for s in range(T) if s <= t and (full or t - s <= Wn)]
                sc = np.array([np.dot(q[b, t, h], k[b, s, j]) / math.sqrt(D) for s in keys])
                w = np.exp(sc - sc.max())
                w /= w.sum()
                y[b, t, h] = sum(wi * v[b, s, j] for wi, s in zip(w, keys))
    return y


@pytest.mark.parametrize("full", [True, False])
def test_attention_matches_loops(full):
    rng = np.random.default_rng(4)
    q = rng.standard_normal((2, 13, 4, 8))
    k = rng.standard_normal((2, 13, 2, 8))
    v = rng.standard_normal((2, 13, 2, 8))
    np.testing.assert_allclose(oracle.attention_fwd(q, k, v, full, 4),
                               _loop_attention(q, k, v, full, 4), atol=1e-13)


def test_attention_causal_equals_sdpa_with_repeated_kv():
    """Full layers = torch SDPA is_causal; GQA = MHA with K/V heads repeated
    contiguously; a window >= T - 1 reduces a short layer to causal."""
    rng = np.random.default_rng(5)
    B, T, H, Hk, D = 2, 37, 6, 2, 16
    q = rng.standard_normal((B, T, H, D))
    k = rng.standard_normal((B, T, Hk, D))
    v = rng.standard_normal((B, T, Hk, D))
    t = lambda a: torch.from_numpy(a).transpose(1, 2)
    kr = t(k).repeat_interleave(H // Hk, dim=1)
    vr = t(v).repeat_interleave(H // Hk, dim=1)
    ref = F.scaled_dot_product_attention(t(q), kr, vr, is_causal=True).transpose(1, 2).numpy()
    np.testing.assert_allclose(oracle.attention_fwd(q, k, v, True, 0), ref, atol=1e-12)
    np.testing.assert_allclose(oracle.attention_fwd(q, k, v, False, T - 1), ref, atol=1e-12)


def test_attention_window_edge_and_degenerate():
    rng = np.random.default_rng(6)
    B, T, D = 1, 20, 8
    q = rng.standard_normal((B, T, 1, D))
    k = rng.standard_normal((B, T, 1, D))
    v = rng.standard_normal((B, T, 1, D))
    m = oracle.visible(T, False, 5)
    assert m[10, 5] and not m[10, 4] and m[10, 10] and not m[10, 11]
    assert m.sum(axis=1).min() >= 1
    # W = 0: every query sees only itself -> y = v
    np.testing.assert_allclose(oracle.attention_fwd(q, k, v, False, 0), v, atol=1e-14)
    # T = 1 -> y = v
    np.testing.assert_allclose(oracle.attention_fwd(q[:, :1], k[:, :1], v[:, :1], True, 0),
                               v[:, :1], atol=1e-14)


def test_attention_bwd_matches_autograd():
    rng = np.random.default_rng(7)
    B, T, H, Hk, D, Wn = 2, 23, 4, 2, 8, 6
    q = rng.standard_normal((B, T, H, D))
    k = rng.standard_normal((B, T, Hk, D))
    v = rng.standard_normal((B, T, Hk, D))
    gy = rng.standard_normal((B, T, H, D))
    for full in (True, False):
        y = oracle.attention_fwd(q, k, v, full, Wn)
        gq, gk, gv = oracle.attention_bwd(q, k, v, y, gy, full, Wn)
        mask = torch.from_numpy(oracle.visible(T, full, Wn))
        qt, kt, vt = (torch.from_numpy(a).requires_grad_() for a in (q, k, v))
        tt = lambda a: a.transpose(1, 2)
        out = F.scaled_dot_product_attention(
            tt(qt), tt(kt).repeat_interleave(H // Hk, 1), tt(vt).repeat_interleave(H // Hk, 1),
            attn_mask=mask)
        out.transpose(1, 2).backward(torch.from_numpy(gy))
        np.testing.assert_allclose(gq, qt.grad.numpy(), atol=1e-12)
        np.testing.assert_allclose(gk, kt.grad.numpy(), atol=1e-12)
        np.testing.assert_allclose(gv, vt.grad.numpy(), atol=1e-12)


# ---------------------------------------------------------------- softcap + CE

def test_softcap_ce_matches_torch():
    rng = np.random.default_rng(8)
    z = rng.standard_normal((9, 50)) * 20
    y = rng.integers(0, 50, 9)
    y[3] = -1
    loss, gz, c = oracle.softcap_ce_fwd_bwd(z, y, 15.0)
    assert np.abs(c).max() <= 15.0
    zt = torch.from_numpy(z).requires_grad_()
    ref = F.cross_entropy(15 * torch.tanh(zt / 15), torch.from_numpy(y), ignore_index=-1)
    ref.backward()
    assert abs(loss - ref.item()) < 1e-13
    np.testing.assert_allclose(gz, zt.grad.numpy(), atol=1e-15)
    # small-z expansion: 15 tanh(z/15) ~ z - z^3/675
    zs = np.array([[1e-3, -2e-3]])
    _, _, cs = oracle.softcap_ce_fwd_bwd(zs, np.array([0]), 15.0)
    np.testing.assert_allclose(cs, zs - zs ** 3 / 675, rtol=1e-12)
    # each valid row's logit gradient sums to zero
    assert np.abs(gz.sum(axis=1)[y >= 0] / (1 - 0)).max() < 1  # bounded
    _, gz0, _ = oracle.softcap_ce_fwd_bwd(np.zeros((4, 10)), np.array([1, 2, 3, -1]), 15.0)
    np.testing.assert_allclose(gz0.sum(axis=1), 0, atol=1e-16)


@pytest.mark.parametrize("name", ["tiny"])
def test_zero_lm_head_gives_ln_vocab(name):
    """All-zero lm_head: every logit is 0, so the loss is ln V exactly and
    the logit gradient is (1/V - onehot) / N."""
    cfg = W.get(name)
    offs, total = oracle.param_offsets(cfg)
    p = W.gen_params(total, cfg.n_layer, 7).astype(np.float64)
    o, s = offs["lm_head"]
    p[o:o + np.prod(s)] = 0
    tok, tgt = W.split_tokens(W.gen_tokens(cfg))
    loss, grads, acts = oracle.forward_backward(cfg, p, tok, tgt, return_acts=True)
    assert abs(loss - math.log(cfg.vocab)) < 1e-12
    assert abs(math.log(512) - 6.2383) < 1e-4
    gz = acts["final"]["gz"]
    N = tgt.size
    ref = np.full_like(gz, 1.0 / cfg.vocab / N)
    ref[np.arange(N), tgt.reshape(-1)] -= 1.0 / N
    np.testing.assert_allclose(gz, ref, atol=1e-17)


def test_init_loss_near_ln_vocab():
    """With N(0, 0.02^2) weights the logits are small; the loss sits near
    ln V + 0.02^2 * C / 2 (a statistical statement, tolerance 1e-2)."""
    cfg = W.get("tiny")
    _, total = oracle.param_offsets(cfg)
    p = W.gen_params(total, cfg.n_layer, W.weight_seed(cfg)).astype(np.float64)
    tok, tgt = W.split_tokens(W.gen_tokens(cfg))
    loss = oracle.forward_loss(cfg, p, tok, tgt)
    assert abs(loss - (math.log(512) + 0.02 ** 2 * 128 / 2)) < 2e-2


# ---------------------------------------------------------------- structure

def test_uniform_attention_closed_form():
    """Wq = Wk = 0 makes q = k = 0 after RoPE and QK-norm, so each query
    averages v over its visible keys; Wg = 0 makes the value-embedding gate
    exactly 1/2. With an identity-like Wo and zero MLP the block output is
    checked against cumulative means, for the short and the full layer."""
    cfg = _tiny(n_layer=2, batch=1)
    offs, total = oracle.param_offsets(cfg)
    p = W.gen_params(total, 2, 11).astype(np.float64)
    P = oracle.unpack(cfg, p)
    for l in range(2):
        P[f"l{l}.q"][...] = 0
        P[f"l{l}.k"][...] = 0
        P[f"l{l}.fc"][...] = 0
    P["l1.veg"][...] = 0
    tok, tgt = W.split_tokens(W.gen_tokens(cfg))
    _, _, acts = oracle.forward_backward(cfg, p, tok, tgt, return_acts=True)
    T, Wn = cfg.seq_len, cfg.short_window
    for l, full in ((0, False), (1, True)):
        c = acts[l]
        xn = c["xn"]
        v = (xn @ P[f"l{l}.v"].T).reshape(T, cfg.n_kv_head, cfg.head_dim)
        if l == 1:
            v = v + 0.5 * P["l1.ve"][tok[0]].reshape(T, cfg.n_kv_head, cfg.head_dim)
        ref = np.zeros((T, cfg.n_head, cfg.head_dim))
        for t in range(T):
            lo = 0 if full else max(0, t - Wn)
            ref[t] = np.repeat(v[lo:t + 1].mean(axis=0), cfg.n_head // cfg.n_kv_head, axis=0)
        np.testing.assert_allclose(c["y"][0], ref, atol=1e-12)
        # the residual stream after the block: xin + y Wo^T (MLP is zero)
        np.testing.assert_allclose(c["xm"], c["xin"] + ref.reshape(T, -1) @ P[f"l{l}.o"].T,
                                   atol=1e-12)
    # the mix: xin = lr * x + l0 * x0 with x0 = wte[tok]
    x0 = P["wte"][tok[0]]
    lr, l0 = P["resid_lambdas"], P["x0_lambdas"]
    np.testing.assert_allclose(acts[0]["xin"], (lr[0] + l0[0]) * x0, rtol=0, atol=1e-15)
    np.testing.assert_allclose(acts[1]["xin"], lr[1] * acts[0]["xm"] + l0[1] * x0,
                               rtol=0, atol=1e-15)


def test_identity_blocks_reduce_to_unigram_model():
    """o = mp = 0 makes every block add nothing, so the loss depends only on
    wte and lm_head through rms, softcap and CE (torch library routines)."""
    cfg = W.get("tiny")
    offs, total = oracle.param_offsets(cfg)
    p = W.gen_params(total, cfg.n_layer, 12).astype(np.float64) * 10
    P = oracle.unpack(cfg, p)
    for l in range(cfg.n_layer):
        P[f"l{l}.o"][...] = 0
        P[f"l{l}.mp"][...] = 0
    P["resid_lambdas"][...] = [0.7, 1.3]
    P["x0_lambdas"][...] = [0.2, 0.5]
    tok, tgt = W.split_tokens(W.gen_tokens(cfg))
    loss = oracle.forward_loss(cfg, p, tok, tgt)
    x0 = torch.from_numpy(P["wte"][tok.reshape(-1)])
    a = (0.7 * 1 + 0.2) * 1.3 + 0.5           # x after two mixes = a * x0
    xf = F.rms_norm(a * x0, (cfg.n_embd,), eps=2.0 ** -23)
    z = xf @ torch.from_numpy(P["lm_head"]).T
    ref = F.cross_entropy(15 * torch.tanh(z / 15), torch.from_numpy(tgt.reshape(-1)).long())
    assert abs(loss - ref.item()) < 1e-12


# ---------------------------------------------------------------- gradients

def _fd_entries(cfg, rng, per_tensor=20):
    offs, total = oracle.param_offsets(cfg)
    idx = []
    for name, (o, s) in offs.items():
        n = int(np.prod(s))
        if name.endswith("lambdas"):
            idx += [o + i for i in range(n)]
        else:
            idx += list(o + rng.choice(n, size=min(per_tensor, n), replace=False))
    return idx


def test_finite_differences_tiny():
    """Central differences in float64 on every lambda and 20 random entries
    of every other tensor. Entries of the embedding tables are drawn from the
    rows the batch uses, where the gradient is not trivially zero."""
    cfg = W.get("tiny")
    offs, total = oracle.param_offsets(cfg)
    p = W.gen_params(total, cfg.n_layer, W.weight_seed(cfg)).astype(np.float64)
    tok, tgt = W.split_tokens(W.gen_tokens(cfg))
    _, g = oracle.forward_backward(cfg, p, tok, tgt)
    rng = np.random.default_rng(9)
    idx = _fd_entries(cfg, rng)
    used = np.unique(tok)
    for name in ("wte", "l1.ve"):
        o, s = offs[name]
        rows = rng.choice(used, 20)
        cols = rng.integers(0, s[1], 20)
        idx += list(o + rows * s[1] + cols)
    h = 1e-5
    worst = 0.0
    for i in idx:
        pp = p.copy(); pp[i] += h
        pm = p.copy(); pm[i] -= h
        fd = (oracle.forward_loss(cfg, pp, tok, tgt) - oracle.forward_loss(cfg, pm, tok, tgt)) / (2 * h)
        err = abs(fd - g[i]) / max(abs(g[i]), 1e-4)
        worst = max(worst, err)
        assert err < 1e-6, (i, fd, g[i])
    assert worst < 1e-6


def _torch_model_loss(cfg, params, tok, tgt, linear=F.linear):
    """The model assembled from torch library ops (rms_norm, SDPA with an
    explicit mask, cross_entropy) for an autograd cross-check. ``linear``
    computes the six block linears (the ve gate and lm_head use F.linear)."""
    L, C, H, Hk, D = cfg.n_layer, cfg.n_embd, cfg.n_head, cfg.n_kv_head, cfg.head_dim
    B, T = tok.shape
    offs, _ = oracle.param_offsets(cfg)
    Pt = {n: params[o:o + int(np.prod(s))].view(*s) for n, (o, s) in offs.items()}
    tk = torch.from_numpy(tok).long()
    eps = cfg.norm_eps
    pos = torch.arange(T, dtype=torch.float64)[:, None]
    inv = cfg.rope_theta ** (-torch.arange(0, D, 2, dtype=torch.float64) / D)
    ang = pos * inv[None]
    cs, sn = torch.cos(ang)[None, :, None, :], torch.sin(ang)[None, :, None, :]

    def rot(x):
        a, b = x[..., :D // 2], x[..., D // 2:]
        return torch.cat([a * cs - b * sn, a * sn + b * cs], -1)

    x0 = F.embedding(tk, Pt["wte"])
    if getattr(cfg, "smear", False):
        # previous token's embedding, zero at position 0 (gate output unused there)
        prev = torch.cat([torch.zeros_like(x0[:, :1]), x0[:, :-1]], 1)
        gate = torch.sigmoid(F.linear(x0, Pt["smear_gate"]))
        x0 = x0 + gate * prev
    x = x0
    cached = None
    for l in range(L):
        if l == L // 2:
            cached = x
        x = Pt["resid_lambdas"][l] * x + Pt["x0_lambdas"][l] * x0
        xn = F.rms_norm(x, (C,), eps=eps)
        q = linear(xn, Pt[f"l{l}.q"]).view(B, T, H, D)
        k = linear(xn, Pt[f"l{l}.k"]).view(B, T, Hk, D)
        v = linear(xn, Pt[f"l{l}.v"]).view(B, T, Hk, D)
        q = F.rms_norm(rot(q), (D,), eps=eps)
        k = F.rms_norm(rot(k), (D,), eps=eps)
        if oracle.layer_has_ve(l, L):
            g = torch.sigmoid(F.linear(xn, Pt[f"l{l}.veg"]))[..., None]
            v = v + g * F.embedding(tk, Pt[f"l{l}.ve"]).view(B, T, Hk, D)
        full = l % 4 == 3 or l == L - 1
        ti = torch.arange(T)
        mask = (ti[None, :] <= ti[:, None])
        if not full:
            mask &= (ti[:, None] - ti[None, :]) <= cfg.short_window
        y = F.scaled_dot_product_attention(
            q.transpose(1, 2), k.transpose(1, 2).repeat_interleave(H // Hk, 1),
            v.transpose(1, 2).repeat_interleave(H // Hk, 1), attn_mask=mask)
        x = x + linear(y.transpose(1, 2).reshape(B, T, H * D), Pt[f"l{l}.o"])
        x = x + linear(F.relu(linear(F.rms_norm(x, (C,), eps=eps), Pt[f"l{l}.fc"])).square(),
                       Pt[f"l{l}.mp"])
    if getattr(cfg, "backout", False):
        x = x - Pt["backout_lambda"][0] * cached
    z = F.linear(F.rms_norm(x, (C,), eps=eps), Pt["lm_head"])
    c = cfg.softcap * torch.tanh(z / cfg.softcap)
    return F.cross_entropy(c.view(B * T, -1), torch.from_numpy(tgt).long().view(-1),
                           ignore_index=-1)


@pytest.mark.parametrize("variant", ["tiny", "tiny_gqa_ignore", "smear_backout",
                                     "smear_backout_L3"])
def test_full_model_matches_torch_autograd(variant):
    cfg = W.get("tiny")
    if variant == "tiny_gqa_ignore":
        cfg = cfg.with_(n_head=4, n_kv_head=2, head_dim=32, n_layer=4, short_window=5)
    if variant.startswith("smear_backout"):
        cfg = cfg.with_(smear=True, backout=True)
    if variant == "smear_backout_L3":
        cfg = cfg.with_(n_layer=3, seq_len=20)
    offs, total = oracle.param_offsets(cfg)
    p = W.gen_params(total, cfg.n_layer, 21).astype(np.float64)
    if cfg.smear:
        p[offs["smear_gate"][0]:][:cfg.n_embd] *= 50     # gates away from 1/2
    if cfg.backout:
        p[offs["backout_lambda"][0]] = 0.5
    tok, tgt = W.split_tokens(W.gen_tokens(cfg))
    if variant == "tiny_gqa_ignore":
        tgt = tgt.copy()
        tgt[0, :5] = -1
    loss, g = oracle.forward_backward(cfg, p, tok, tgt)
    pt = torch.from_numpy(p.copy()).requires_grad_()
    ref = _torch_model_loss(cfg, pt, tok, tgt)
    ref.backward()
    assert abs(loss - ref.item()) < 1e-12 * abs(loss)
    ref_g = pt.grad.numpy()
    for name, (o, s) in offs.items():
        n = int(np.prod(s))
        a, b = g[o:o + n], ref_g[o:o + n]
        assert np.linalg.norm(a - b) <= 1e-10 * max(np.linalg.norm(b), 1e-30), name


def test_fp32_mode_close_to_fp64():
    cfg = W.get("tiny")
    _, total = oracle.param_offsets(cfg)
    p = W.gen_params(total, cfg.n_layer, 5)
    tok, tgt = W.split_tokens(W.gen_tokens(cfg))
    l64, g64 = oracle.forward_backward(cfg, p.astype(np.float64), tok, tgt)
    l32, g32 = oracle.forward_backward(cfg, p, tok, tgt, dtype=np.float32)
    assert abs(l32 - l64) / l64 < 1e-6
    assert np.linalg.norm(g32 - g64) / np.linalg.norm(g64) < 1e-5


# ---------------------------------------------------------------- fp8

@pytest.mark.parametrize("fmt,tdt", [("e4m3", torch.float8_e4m3fn), ("e5m2", torch.float8_e5m2)])
def test_fp8_rounding_matches_torch(fmt, tdt):
    codes = torch.arange(256, dtype=torch.uint8).view(tdt).double().numpy()
    codes = codes[np.isfinite(codes)]
    np.testing.assert_array_equal(oracle.fp8.round_fp8(codes, fmt), codes)
    fmax = oracle.fp8.FORMATS[fmt][2]
    rng = np.random.default_rng(10)
    x = np.concatenate([rng.standard_normal(20000) * s for s in (1e-5, 1e-2, 1, 30, 3000)])
    x = np.clip(x, -fmax, fmax)
    ref = torch.from_numpy(x).to(tdt).double().numpy()
    np.testing.assert_array_equal(oracle.fp8.round_fp8(x, fmt), ref)
    # saturation
    assert oracle.fp8.round_fp8(np.array([1e9, -1e9]), fmt).tolist() == [fmax, -fmax]


def test_fp8_qdq_scaling():
    rng = np.random.default_rng(11)
    x = rng.standard_normal(1000)
    q = oracle.fp8.qdq(x, "e4m3")
    i = np.argmax(np.abs(x))
    assert abs(q[i] - x[i]) <= 1e-6 * abs(x[i])        # amax maps to +-fmax exactly
    assert np.max(np.abs(q - x)) <= np.max(np.abs(x)) * 2.0 ** -4
    assert np.all(oracle.fp8.qdq(np.zeros(5), "e5m2") == 0)


@pytest.mark.parametrize("fmt,tdt", [("e4m3", torch.float8_e4m3fn), ("e5m2", torch.float8_e5m2)])
def test_fp8_encode_decode_all_codes(fmt, tdt):
    """Byte codes and values agree with torch's float8 dtypes on every
    finite code (library)."""
    codes = torch.arange(256, dtype=torch.uint8)
    vals = codes.view(tdt).double().numpy()
    ok = np.isfinite(vals)
    np.testing.assert_array_equal(oracle.fp8.encode(vals[ok], fmt), codes.numpy()[ok])
    np.testing.assert_array_equal(oracle.fp8.decode(codes.numpy()[ok], fmt), vals[ok])


def _torch_codes(x, fmt, tdt):
    """Per-tensor codes from torch: fp32 scale fmax / amax, fp32 product,
    clamp, torch's round-to-nearest-even float8 cast."""
    fmax = oracle.fp8.FORMATS[fmt][2]
    xt = torch.from_numpy(np.asarray(x)).float()
    amax = xt.abs().max()
    s = torch.tensor(fmax, dtype=torch.float32) / amax if amax > 0 else torch.tensor(1.0)
    return (xt * s).clamp(-fmax, fmax).to(tdt).view(torch.uint8).numpy(), s.item()


@pytest.mark.parametrize("fmt,tdt", [("e4m3", torch.float8_e4m3fn), ("e5m2", torch.float8_e5m2)])
def test_fp8_quantize_codes_match_torch(fmt, tdt):
    rng = np.random.default_rng(12)
    for scale in (1e-3, 1.0, 40.0):
        x = (rng.standard_normal(50000) * scale).astype(np.float32)
        x[rng.integers(0, x.size, 50)] = 0.0
        codes, s = oracle.fp8.quantize(x, fmt)
        ref, s_ref = _torch_codes(x, fmt, tdt)
        assert np.float32(s) == np.float32(s_ref)
        np.testing.assert_array_equal(codes, ref)
        # the element of largest magnitude maps to +-fmax
        i = np.argmax(np.abs(x))
        assert abs(oracle.fp8.decode(codes[i:i + 1], fmt)[0]) == oracle.fp8.FORMATS[fmt][2]
    # all-zero tensor: scale 1, all codes 0
    codes, s = oracle.fp8.quantize(np.zeros(7, np.float32), fmt)
    assert s == 1.0 and not codes.any()


class _FakeQuantLinear(torch.autograd.Function):
    """y = Q(x) Q(W)^T; g_x = Q(g_y) Q(W); g_W = Q(g_y)^T Q(x), with Q the
    per-tensor quantise-dequantise built from torch's float8 casts."""

    @staticmethod
    def _q(t, fmt, tdt):
        codes, s = _torch_codes(t.detach().numpy(), fmt, tdt)
        v = torch.from_numpy(codes.copy()).view(tdt).double()
        return (v / s).reshape(t.shape)

    @staticmethod
    def forward(ctx, x, w):
        ctx.save_for_backward(x, w)
        e4 = torch.float8_e4m3fn
        return _FakeQuantLinear._q(x, "e4m3", e4) @ _FakeQuantLinear._q(w, "e4m3", e4).T

    @staticmethod
    def backward(ctx, gy):
        x, w = ctx.saved_tensors
        e4, e5 = torch.float8_e4m3fn, torch.float8_e5m2
        q = _FakeQuantLinear._q
        g = q(gy.reshape(-1, gy.shape[-1]), "e5m2", e5)
        xq = q(x.reshape(-1, x.shape[-1]), "e4m3", e4)
        wq = q(w, "e4m3", e4)
        return (g @ wq).reshape(x.shape), g.T @ xq


@pytest.mark.parametrize("variant", ["tiny", "tiny_gqa"])
def test_fp8_model_matches_torch_fake_quant(variant):
    """The oracle's fp8 mode against torch autograd through a fake-quant
    linear whose rounding is torch's own float8 cast."""
    cfg = W.get("tiny").with_(fp8_linears=True)
    if variant == "tiny_gqa":
        cfg = cfg.with_(n_head=4, n_kv_head=2, head_dim=32, n_layer=3, short_window=7)
    offs, total = oracle.param_offsets(cfg)
    p = W.gen_params(total, cfg.n_layer, 23).astype(np.float64)
    tok, tgt = W.split_tokens(W.gen_tokens(cfg))
    loss, g = oracle.forward_backward(cfg, p, tok, tgt)
    pt = torch.from_numpy(p.copy()).requires_grad_()
    ref = _torch_model_loss(cfg, pt, tok, tgt, linear=_FakeQuantLinear.apply)
    ref.backward()
    assert abs(loss - ref.item()) < 1e-9 * abs(loss)
    ref_g = pt.grad.numpy()
    for name, (o, s) in offs.items():
        n = int(np.prod(s))
        a, b = g[o:o + n], ref_g[o:o + n]
        assert np.linalg.norm(a - b) <= 1e-8 * max(np.linalg.norm(b), 1e-30), name
    # fp8 really changes the result relative to the unquantised model
    l0, _ = oracle.forward_backward(cfg, p, tok, tgt, fp8=False)
    assert abs(l0 - loss) > 1e-6


def test_round_bf16_matches_torch():
    """Ties to even on exact halfway cases and on random values (library)."""
    rng = np.random.default_rng(13)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    ties = x.view(np.uint32).copy()
    ties[:5000] = (ties[:5000] & 0xFFFF0000) | 0x8000    # exactly halfway
    x = ties.view(np.float32)
    ref = torch.from_numpy(x.copy()).bfloat16().float().numpy()
    np.testing.assert_array_equal(oracle.fp8.round_bf16(x), ref)


def test_fp8_round_variant_only_touches_quantiser_inputs():
    """fp8_round="bf16" changes an fp8 run but not an unquantised one."""
    cfg = W.get("tiny").with_(fp8_linears=True)
    _, total = oracle.param_offsets(cfg)
    p = W.gen_params(total, cfg.n_layer, 3)
    tok, tgt = W.split_tokens(W.gen_tokens(cfg))
    l0, g0 = oracle.forward_backward(cfg, p, tok, tgt, dtype=np.float32, fp8=False)
    l1, g1 = oracle.forward_backward(cfg, p, tok, tgt, dtype=np.float32, fp8=False, fp8_round="bf16")
    assert l0 == l1 and np.array_equal(g0, g1)
    l2, _ = oracle.forward_backward(cfg, p, tok, tgt, dtype=np.float32)
    l3, _ = oracle.forward_backward(cfg, p, tok, tgt, dtype=np.float32, fp8_round="bf16")
    assert l2 != l3 and abs(l2 - l3) < 1e-2 * abs(l2)


# ---------------------------------------------------------------- Smear / Backout

def _variant_params(cfg, base_cfg, p_base, w_smear=None, lam_b=None):
    """Parameters of a variant config: the base tensors copied by name, the
    variant's own tensors set from the arguments."""
    offs_v, total_v = oracle.param_offsets(cfg)
    offs_b, _ = oracle.param_offsets(base_cfg)
    p = np.zeros(total_v)
    for name, (o, s) in offs_b.items():
        n = int(np.prod(s))
        p[offs_v[name][0]:offs_v[name][0] + n] = p_base[o:o + n]
    if "smear_gate" in offs_v:
        o = offs_v["smear_gate"][0]
        p[o:o + cfg.n_embd] = w_smear
    if "backout_lambda" in offs_v:
        p[offs_v["backout_lambda"][0]] = lam_b
    return p


def test_variant_layout():
    base = W.get("tiny")
    cfg = base.with_(smear=True, backout=True)
    offs, total = oracle.param_offsets(cfg)
    assert total == 590_084 + 128 + 1
    assert offs["smear_gate"] == (offs["lm_head"][0] + 512 * 128, (1, 128))
    assert offs["backout_lambda"] == (offs["smear_gate"][0] + 128, (1,))
    assert offs["resid_lambdas"][0] == offs["backout_lambda"][0] + 1
    assert [n for n, _ in oracle.layout(cfg)][-2:] == ["resid_lambdas", "x0_lambdas"]
    assert oracle.backout_layer(12) == 6 and oracle.backout_layer(1) == 0


def test_smear_closed_form():
    """With w = 0 every gate is 1/2: x0[t] = e[t] + e[t-1] / 2 for t >= 1,
    x0[0] = e[0] (no previous token)."""
    cfg = W.get("tiny").with_(smear=True)
    offs, total = oracle.param_offsets(cfg)
    p = W.gen_params(total, cfg.n_layer, 4).astype(np.float64)
    o = offs["smear_gate"][0]
    p[o:o + cfg.n_embd] = 0
    tok, tgt = W.split_tokens(W.gen_tokens(cfg))
    _, _, acts = oracle.forward_backward(cfg, p, tok, tgt, return_acts=True)
    wte = oracle.unpack(cfg, p)["wte"]
    e = wte[tok]                                          # [B, T, C]
    want = e.copy()
    want[:, 1:] += 0.5 * e[:, :-1]
    np.testing.assert_allclose(acts[0]["x"].reshape(e.shape), want, rtol=0, atol=1e-15)


def test_smear_single_position_is_base_model():
    """seq_len 1: no token has a predecessor, so Smear changes nothing (loss
    and every shared gradient equal the base model's; the gate's is 0)."""
    base = W.get("tiny").with_(seq_len=1, batch=6)
    cfg = base.with_(smear=True)
    _, tb = oracle.param_offsets(base)
    pb = W.gen_params(tb, base.n_layer, 8).astype(np.float64)
    pv = _variant_params(cfg, base, pb, w_smear=np.linspace(-3, 3, base.n_embd))
    tok, tgt = W.split_tokens(W.gen_tokens(base.with_(seq_len=2)))
    tok, tgt = tok[:, :1].copy(), tgt[:, :1].copy()
    lb, gb = oracle.forward_backward(base, pb, tok, tgt)
    lv, gv = oracle.forward_backward(cfg, pv, tok, tgt)
    assert lv == lb
    offs_v, _ = oracle.param_offsets(cfg)
    for name, (o, s) in oracle.param_offsets(base)[0].items():
        n = int(np.prod(s))
        np.testing.assert_array_equal(gv[offs_v[name][0]:offs_v[name][0] + n], gb[o:o + n])
    o = offs_v["smear_gate"][0]
    assert not np.any(gv[o:o + cfg.n_embd])


def test_backout_zero_lambda_is_base_model():
    base = W.get("tiny")
    cfg = base.with_(backout=True)
    _, tb = oracle.param_offsets(base)
    pb = W.gen_params(tb, base.n_layer, 9).astype(np.float64)
    pv = _variant_params(cfg, base, pb, lam_b=0.0)
    tok, tgt = W.split_tokens(W.gen_tokens(base))
    lb, gb = oracle.forward_backward(base, pb, tok, tgt)
    lv, gv = oracle.forward_backward(cfg, pv, tok, tgt)
    assert lv == lb
    offs_v, _ = oracle.param_offsets(cfg)
    for name, (o, s) in oracle.param_offsets(base)[0].items():
        n = int(np.prod(s))
        np.testing.assert_allclose(gv[offs_v[name][0]:offs_v[name][0] + n], gb[o:o + n],
                                   rtol=0, atol=1e-15)
    assert gv[offs_v["backout_lambda"][0]] != 0


def test_backout_identity_blocks_closed_form():
    """o = mp = 0: the stream after k blocks is a_k * x0 with
    a_k = lr_k a_{k-1} + l0_k, a_0 = 1. With 3 layers the cached stream is
    the one entering layer 1 (a_1 x0), so the final norm sees
    (a_3 - lambda a_1) x0; the loss then follows from torch routines."""
    cfg = W.get("tiny").with_(n_layer=3, backout=True)
    offs, total = oracle.param_offsets(cfg)
    p = W.gen_params(total, cfg.n_layer, 12).astype(np.float64) * 10
    P = oracle.unpack(cfg, p)
    for l in range(cfg.n_layer):
        P[f"l{l}.o"][...] = 0
        P[f"l{l}.mp"][...] = 0
    lr, l0 = [0.7, 1.3, 0.9], [0.2, 0.5, -0.4]
    P["resid_lambdas"][...] = lr
    P["x0_lambdas"][...] = l0
    P["backout_lambda"][...] = 0.75
    a = [1.0]
    for k in range(3):
        a.append(lr[k] * a[-1] + l0[k])
    coef = a[3] - 0.75 * a[1]
    tok, tgt = W.split_tokens(W.gen_tokens(cfg))
    loss = oracle.forward_loss(cfg, p, tok, tgt)
    x0 = torch.from_numpy(P["wte"][tok.reshape(-1)])
    xf = F.rms_norm(coef * x0, (cfg.n_embd,), eps=2.0 ** -23)
    z = xf @ torch.from_numpy(P["lm_head"]).T
    ref = F.cross_entropy(15 * torch.tanh(z / 15), torch.from_numpy(tgt.reshape(-1)).long())
    assert abs(loss - ref.item()) < 1e-12


def test_finite_differences_smear_backout():
    """Central differences on the two variant tensors (every smear-gate
    entry, lambda), the lambdas and 8 entries of every other tensor."""
    cfg = W.get("tiny").with_(smear=True, backout=True, n_layer=3, seq_len=24)
    offs, total = oracle.param_offsets(cfg)
    p = W.gen_params(total, cfg.n_layer, 31).astype(np.float64)
    o = offs["smear_gate"][0]
    p[o:o + cfg.n_embd] *= 50
    p[offs["backout_lambda"][0]] = 0.5
    tok, tgt = W.split_tokens(W.gen_tokens(cfg))
    _, g = oracle.forward_backward(cfg, p, tok, tgt)
    rng = np.random.default_rng(3)
    idx = list(range(o, o + cfg.n_embd, 7)) + [offs["backout_lambda"][0]]
    for name, (oo, s) in offs.items():
        n = int(np.prod(s))
        if name.endswith("lambdas"):
            idx += [oo + i for i in range(n)]
        elif name not in ("smear_gate", "backout_lambda"):
            idx += list(oo + rng.choice(n, size=min(8, n), replace=False))
    used = np.unique(tok)
    ow = offs["wte"][0]
    idx += list(ow + rng.choice(used, 12) * cfg.n_embd + rng.integers(0, cfg.n_embd, 12))
    h = 1e-5
    for i in idx:
        pp = p.copy(); pp[i] += h
        pm = p.copy(); pm[i] -= h
        fd = (oracle.forward_loss(cfg, pp, tok, tgt) - oracle.forward_loss(cfg, pm, tok, tgt)) / (2 * h)
        assert abs(fd - g[i]) <= 1e-6 * max(abs(g[i]), 1e-4), (i, fd, g[i])


# ---------------------------------------------------------------- decode attention

def _decode_case(B=3, H=4, Hk=2, D=16, Tmax=40, seed=0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, D))
    k = rng.standard_normal((B, Tmax, Hk, D))
    v = rng.standard_normal((B, Tmax, Hk, D))
    seqlen = rng.integers(1, Tmax + 1, B)
    return q, k, v, seqlen


@pytest.mark.parametrize("window", [None, 0, 5, 100])
def test_decode_attention_matches_sdpa(window):
    """Against torch SDPA (float64) on the cached rows, with the window as
    an explicit boolean mask."""
    q, k, v, seqlen = _decode_case(seed=1)
    out = oracle.decode.decode_attention(q, k, v, seqlen, window)
    B, H, D = q.shape
    G = H // k.shape[2]
    for b in range(B):
        t = int(seqlen[b]) - 1
        s = np.arange(k.shape[1])
        mask = s <= t
        if window is not None:
            mask &= (t - s) <= window
        kb = torch.from_numpy(k[b]).transpose(0, 1).repeat_interleave(G, 0)   # [H, Tmax, D]
        vb = torch.from_numpy(v[b]).transpose(0, 1).repeat_interleave(G, 0)
        ref = F.scaled_dot_product_attention(torch.from_numpy(q[b])[:, None, :], kb, vb,
                                             attn_mask=torch.from_numpy(mask)[None, None, :])
        np.testing.assert_allclose(out[b], ref[:, 0].numpy(), rtol=1e-12, atol=1e-12)


def test_decode_attention_brute_force_and_invariants():
    q, k, v, seqlen = _decode_case(B=2, H=2, Hk=1, D=4, Tmax=6, seed=2)
    seqlen = np.array([6, 3])
    out = oracle.decode.decode_attention(q, k, v, seqlen, window=2)
    # brute force with scalar loops: sequence 0 sees positions 3, 4, 5
    for h in range(2):
        w = [math.exp(sum(q[0, h, d] * k[0, s, 0, d] for d in range(4)) / 2.0) for s in (3, 4, 5)]
        ref = [sum(w[i] * v[0, s, 0, d] for i, s in enumerate((3, 4, 5))) / sum(w)
               for d in range(4)]
        np.testing.assert_allclose(out[0, h], ref, rtol=1e-12)
    # one visible key: the output is that value row
    one = oracle.decode.decode_attention(q, k, v, np.array([6, 3]), window=0)
    np.testing.assert_array_equal(one[0], np.repeat(v[0, 5], 2, 0).reshape(2, 4))
    # a window at least as long as the sequence is the full causal case
    np.testing.assert_allclose(oracle.decode.decode_attention(q, k, v, seqlen, 10),
                               oracle.decode.decode_attention(q, k, v, seqlen, None), rtol=0,
                               atol=0)
    # equal value rows: the output is that row whatever the scores
    v2 = np.broadcast_to(v[:, :1], v.shape)
    o2 = oracle.decode.decode_attention(q, k, v2, seqlen, None)
    np.testing.assert_allclose(o2[1, 0], v[1, 0, 0], rtol=1e-12)


def test_kv_cache_append_by_hand():
    """Every written element checked against the qkv column it comes from,
    element by element; rows outside [0, max_len) are left alone."""
    B, n_new, H, Hk, D, Tmax = 2, 3, 4, 2, 8, 5
    qkv = np.arange(B * n_new * (H + 2 * Hk) * D, dtype=np.float64).reshape(B * n_new, -1)
    k = np.full((B, Tmax, Hk, D), -1.0)
    v = np.full((B, Tmax, Hk, D), -2.0)
    pos = np.array([1, 4])                   # sequence 1: only its first new token fits
    oracle.decode.kv_cache_append(qkv, pos, k, v, H, Hk, D)
    for b in range(B):
        for p in range(Tmax):
            i = p - pos[b]
            for j in range(Hk):
                for d in range(D):
                    if 0 <= i < n_new:
                        assert k[b, p, j, d] == qkv[b * n_new + i, H * D + j * D + d]
                        assert v[b, p, j, d] == qkv[b * n_new + i, (H + Hk) * D + j * D + d]
                    else:
                        assert k[b, p, j, d] == -1.0 and v[b, p, j, d] == -2.0


# ---------------------------------------------------------------- MuonAdamW

def test_adamw_matches_torch():
    rng = np.random.default_rng(5)
    p0 = rng.standard_normal(50)
    p = p0.copy(); m = np.zeros(50); v = np.zeros(50)
    pt = torch.tensor(p0, requires_grad=True)
    opt = torch.optim.AdamW([pt], lr=0.3, betas=(0.8, 0.95), eps=1e-10, weight_decay=0.1)
    for t in range(1, 5):
        g = rng.standard_normal(50)
        oracle.optim.adamw_update(p, g, m, v, 0.3, t, 0.8, 0.95, 1e-10, wd=0.1)
        pt.grad = torch.from_numpy(g.copy())
        opt.step()
        np.testing.assert_allclose(p, pt.detach().numpy(), rtol=1e-12, atol=1e-12)


def _polar(Mx):
    U, _, Vt = np.linalg.svd(Mx, full_matrices=False)
    return U @ Vt


@pytest.mark.parametrize("shape", [(8, 8), (6, 20), (20, 6)])
def test_newton_schulz_cubic_converges_to_polar_factor(shape):
    """With the cubic coefficients (1.5, -0.5, 0) the iteration converges to
    the orthogonal polar factor U V^T of the SVD G = U S V^T."""
    rng = np.random.default_rng(6)
    U, _ = np.linalg.qr(rng.standard_normal((shape[0], min(shape))))
    V, _ = np.linalg.qr(rng.standard_normal((shape[1], min(shape))))
    G = U @ np.diag(np.linspace(1.0, 3.0, min(shape))) @ V.T      # condition number 3
    X = oracle.optim.newton_schulz(G, 1.5, -0.5, 0.0, 60)
    np.testing.assert_allclose(X, _polar(G), atol=1e-10)


def test_newton_schulz_quintic_keeps_singular_vectors():
    """The default quintic iteration maps every singular value of a
    well-spread spectrum into a band around 1 and keeps the singular
    vectors: U^T X V is diagonal with entries in (0.6, 1.3)."""
    rng = np.random.default_rng(7)
    U, _ = np.linalg.qr(rng.standard_normal((16, 16)))
    V, _ = np.linalg.qr(rng.standard_normal((48, 16)))
    G = U @ np.diag(np.geomspace(0.05, 5.0, 16)) @ V.T
    d = oracle.optim.DEFAULTS
    X = oracle.optim.newton_schulz(G, d["ns_a"], d["ns_b"], d["ns_c"], d["ns_steps"])
    D = U.T @ X @ V
    assert np.abs(D - np.diag(np.diag(D))).max() < 1e-10
    assert np.all(np.diag(D) > 0.6) and np.all(np.diag(D) < 1.3)


def test_muon_two_steps_closed_form():
    """Orthogonal gradients Q1 then Q2, Nesterov momentum mu, many cubic NS
    steps: the second update direction is the polar factor of
    (1 + mu) Q2 + mu^2 Q1, the first is Q1; tall matrices get
    sqrt(rows / cols)."""
    rng = np.random.default_rng(8)
    Q1, _ = np.linalg.qr(rng.standard_normal((12, 4)))
    Q2, _ = np.linalg.qr(rng.standard_normal((12, 4)))
    p0 = rng.standard_normal((12, 4))
    p, buf = p0.copy(), np.zeros((12, 4))
    mu, lr, wd = 0.9, 0.1, 0.2
    oracle.optim.muon_update(p, Q1, buf, lr, mu, True, wd, 1.5, -0.5, 0.0, 80)
    oracle.optim.muon_update(p, Q2, buf, lr, mu, True, wd, 1.5, -0.5, 0.0, 80)
    s = np.sqrt(12 / 4)
    want = (p0 * (1 - lr * wd) - lr * s * Q1) * (1 - lr * wd) - lr * s * _polar((1 + mu) * Q2 + mu * mu * Q1)
    np.testing.assert_allclose(p, want, atol=1e-9)


def test_optimizer_groups():
    cfg = W.get("tiny").with_(smear=True, backout=True)
    g = {n: oracle.optim.group(n) for n in oracle.param_offsets(cfg)[0]}
    assert g["l0.q"] == g["l1.mp"] == ("muon", "lr_matrix")
    assert g["wte"] == g["l1.ve"] == ("adamw", "lr_embed")
    assert g["lm_head"] == ("adamw", "lr_unembed")
    assert g["resid_lambdas"] == g["l1.veg"] == g["smear_gate"] == g["backout_lambda"] == \
        ("adamw", "lr_scalar")


def test_optimizer_step_matches_torch_groups_and_muon_closed_form():
    """The assembled MuonAdamW step (oracle.optim.optimizer_step) over three
    steps on the small config with Smear and Backout, a schedule multiplier
    0.7 and weight decay 0.28 (report, optimizer and schedule blocks):
      * AdamW tensors equal torch.optim.AdamW run with one param group per
        rate (embedding rate for wte and the value-embedding tables,
        unembedding rate for lm_head, scalar rate for the rest), each rate
        times the multiplier, and no weight decay;
      * Muon tensors follow a closed form: every step's gradient is
        U diag(s_t) V^T with fixed orthonormal U, V and s_t in [1, 3], so the
        momentum buffer is mu buf + g and the Nesterov update u = g + mu buf
        share U, V, and the orthogonalised update is exactly U V^T (cubic
        Newton-Schulz, run to convergence); p <- p (1 - lr wd) - lr
        sqrt(max(1, rows / cols)) U V^T.
    Decay on an AdamW tensor, a dropped multiplier, a wrong rate key or a
    wrong step counter each fail this test."""
    cfg = W.get("tiny").with_(smear=True, backout=True)
    names, total = oracle.param_offsets(cfg)
    rng = np.random.default_rng(11)
    p = rng.standard_normal(total) * 0.1
    m = np.zeros(total)
    v = np.zeros(total)
    hp = dict(lr_mult=0.7, weight_decay=0.28, ns_a=1.5, ns_b=-0.5, ns_c=0.0, ns_steps=60,
              momentum=0.9, nesterov=True, beta1=0.85, beta2=0.99, eps=1e-9)
    d = dict(oracle.optim.DEFAULTS, **hp)
    lay = {n: (o, shp) for n, (o, shp) in names.items()}
    rate_key = {"wte": "lr_embed", "lm_head": "lr_unembed"}
    muon, groups = [], {"lr_embed": [], "lr_unembed": [], "lr_scalar": []}
    tparams = {}
    for n, (o, shp) in lay.items():
        leaf = n.split(".")[-1]
        if leaf in ("q", "k", "v", "o", "fc", "mp"):
            muon.append(n)
            continue
        key = "lr_embed" if leaf == "ve" else rate_key.get(n, "lr_scalar")
        t = torch.tensor(p[o:o + int(np.prod(shp))].copy(), requires_grad=True)
        tparams[n] = t
        groups[key].append(t)
    opt = torch.optim.AdamW([dict(params=ps, lr=d[k] * 0.7) for k, ps in groups.items() if ps],
                            betas=(0.85, 0.99), eps=1e-9, weight_decay=0.0)
    # fixed singular vectors per Muon matrix
    UV = {}
    for n in muon:
        o, (r, c) = lay[n]
        k = min(r, c)
        U, _ = np.linalg.qr(rng.standard_normal((r, k)))
        V, _ = np.linalg.qr(rng.standard_normal((c, k)))
        UV[n] = (U, V, k)
    want = {n: p[lay[n][0]:lay[n][0] + int(np.prod(lay[n][1]))].reshape(lay[n][1]).copy()
            for n in muon}
    want_buf = {n: np.zeros(lay[n][1]) for n in muon}
    lr_m = d["lr_matrix"] * 0.7
    for t in range(1, 4):
        g = rng.standard_normal(total) * 0.01
        for n in muon:
            o, shp = lay[n]
            U, V, k = UV[n]
            G = U @ np.diag(rng.uniform(1.0, 3.0, k)) @ V.T
            g[o:o + G.size] = G.ravel()
            want_buf[n] = 0.9 * want_buf[n] + G
            scale = max(1.0, shp[0] / shp[1]) ** 0.5
            want[n] = want[n] * (1 - lr_m * 0.28) - lr_m * scale * (U @ V.T)
        oracle.optim.optimizer_step(cfg, p, g, m, v, t, **hp)
        for n, tp in tparams.items():
            o = lay[n][0]
            tp.grad = torch.from_numpy(g[o:o + tp.numel()].copy())
        opt.step()
    for n, tp in tparams.items():
        o = lay[n][0]
        sl = slice(o, o + tp.numel())
        np.testing.assert_allclose(p[sl], tp.detach().numpy(), rtol=1e-11, atol=1e-12, err_msg=n)
        st = opt.state[tp]
        np.testing.assert_allclose(m[sl], st["exp_avg"].numpy(), rtol=1e-11, atol=1e-14, err_msg=n)
        np.testing.assert_allclose(v[sl], st["exp_avg_sq"].numpy(), rtol=1e-11, atol=1e-16,
                                   err_msg=n)
    for n in muon:
        o, shp = lay[n]
        sl = slice(o, o + int(np.prod(shp)))
        np.testing.assert_allclose(p[sl].reshape(shp), want[n], atol=1e-9, err_msg=n)
        np.testing.assert_allclose(m[sl].reshape(shp), want_buf[n], atol=1e-12, err_msg=n)
