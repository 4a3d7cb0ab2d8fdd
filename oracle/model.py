"""Plain CPU forward + backward of the nanochat GPT step (test infrastructure).

Everything here is the textbook definition written out with NumPy array
operations: no tiling, no fusion, no reordering. Attention materialises the
full masked score matrix. The backward is derived by hand from the forward
below (chain rule, one formula per forward step) and is pinned by finite
differences and by an independent autograd run in the tests.

Precision: the caller picks the array dtype. float64 is used for the small
config; float32 with float64 accumulation of row statistics, the loss and
the lambda / gate reductions is used for the large ones.

What the pages fix, and the readings taken where they do not
(page titles abbreviated: "report" = NanoChat基础训练报告; "additions" =
Nanochat在nanoGPT之上的新增功能; "overview" = nanochat — 架构与原理):

* Parameter-free RMSNorm replaces LayerNorm (additions, section 1 table,
  normalisation row). eps is not given; eps = 2^-23 (a config value).
* Separate c_q, c_k, c_v, c_proj without bias (additions table, attention
  and bias rows; report, architecture block).
* RoPE without learned positions (additions table and notes). The base and
  the pairing are not given: base 10000 and half-split pairs (i, i + D/2).
* QK-norm after RoPE (additions table): parameter-free RMSNorm over D.
* GQA with n_kv_head <= n_head (additions table and notes); query head h
  reads KV head floor(h / (n_head / n_kv_head)).
* Sliding window per layer in an SSSL pattern, short = 1/4 of the context,
  last layer always full (additions notes; the table's "SSSSL" is read as
  the notes' SSSL). Key s is visible to query t iff s <= t and, on short
  layers, t - s <= W.
* Value embeddings on alternating layers, last included (additions notes;
  report: odd layers of 12). v <- v + gate * ve. The gate's form is not
  given: gate = sigmoid(xn . Wg[j]) per token and KV head j (parity unpinned
  with respect to the pages).
* Per-layer resid_lambdas and x0 lambdas (additions table): at the start of
  every block, x <- lambda_r[l] * x + lambda_0[l] * x0.
* ReLU^2 MLP, hidden 4C, no bias (additions table and notes).
* Untied lm_head; tanh logit softcap with range +-15 (additions table).
* Cross-entropy averaged over targets that are not -1 (overview section 4,
  the -1 ignore index).
* Attention scale 1/sqrt(D).

Model variants (workload flags ``smear`` and ``backout``; "additions",
feature table rows Smear and Backout and the notes on them):

* Smear: x <- x + sigmoid(gate(x)) * x_prev at the embedding. Readings:
  gate is a bias-free linear map C -> 1 ("smear_gate" [1, C]) of the
  current token's embedding; x_prev is the previous token's embedding in
  the same sequence (before smearing); position 0 of a sequence has no
  previous token and is left unchanged; the smeared embedding is the x0
  the blocks mix in.
* Backout: the residual stream is cached at the middle layer and
  lambda * x_backout is subtracted before the final norm. Readings: the
  cached stream is the one entering layer L // 2 (after the first L // 2
  blocks); lambda is one learnable scalar ("backout_lambda" [1]); its
  initial value (the table's "half") is the caller's.
"""
from __future__ import annotations

import numpy as np

from . import fp8 as _fp8


# --------------------------------------------------------------------------
# Layer patterns and parameter layout
# --------------------------------------------------------------------------

def layer_is_full(l: int, L: int) -> bool:
    """SSSL tiled over depth (three short-window layers, then one full
    layer), with the last layer forced full ("additions", notes on the
    sliding window)."""
    return (l % 4 == 3) or (l == L - 1)


def layer_has_ve(l: int, L: int) -> bool:
    """Value embeddings on every other layer counted back from the last one,
    which always has one ("additions", notes on value residuals); this gives
    the odd layers 1..11 of the d12 model ("report", architecture block)."""
    return (l % 2) == ((L - 1) % 2)


def layout(cfg):
    """Canonical flat order of the trainable tensors: name and shape.

    Linear weights are [out, in] (y = x W^T). The value-embedding table of a
    layer is [vocab, n_kv_head * head_dim] because it is added to v; its gate
    is [n_kv_head, n_embd]. With these shapes the d12 total is 286,288,920
    and the non-embedding total (everything but wte) 261,123,096, the
    286.3M / 261.1M of the "report" architecture block.
    """
    C, H, Hk, D = cfg.n_embd, cfg.n_head, cfg.n_kv_head, cfg.head_dim
    F, V, L = cfg.mlp_hidden, cfg.vocab, cfg.n_layer
    out = [("wte", (V, C))]
    for l in range(L):
        out += [(f"l{l}.q", (H * D, C)), (f"l{l}.k", (Hk * D, C)),
                (f"l{l}.v", (Hk * D, C)), (f"l{l}.o", (C, H * D)),
                (f"l{l}.fc", (F, C)), (f"l{l}.mp", (C, F))]
        if layer_has_ve(l, L):
            out += [(f"l{l}.ve", (V, Hk * D)), (f"l{l}.veg", (Hk, C))]
    out += [("lm_head", (V, C))]
    if getattr(cfg, "smear", False):
        out += [("smear_gate", (1, C))]
    if getattr(cfg, "backout", False):
        out += [("backout_lambda", (1,))]
    out += [("resid_lambdas", (L,)), ("x0_lambdas", (L,))]
    return out


def param_offsets(cfg):
    """name -> (offset, shape), and the total element count."""
    offs, o = {}, 0
    for name, shape in layout(cfg):
        offs[name] = (o, shape)
        o += int(np.prod(shape))
    return offs, o


def unpack(cfg, flat):
    """name -> view of ``flat`` with the tensor's shape."""
    offs, total = param_offsets(cfg)
    assert flat.size == total, (flat.size, total)
    return {n: flat[o:o + int(np.prod(s))].reshape(s) for n, (o, s) in offs.items()}


# --------------------------------------------------------------------------
# Step functions
# --------------------------------------------------------------------------

def rms_fwd(x, eps):
    """Parameter-free RMSNorm over the last axis: y = x / sqrt(mean(x^2) + eps).
    Returns y and r = 1 / sqrt(mean(x^2) + eps) (shape [..., 1])."""
    ms = np.mean(np.square(x), axis=-1, keepdims=True, dtype=np.float64)
    r = (1.0 / np.sqrt(ms + eps)).astype(x.dtype)
    return x * r, r


def rms_bwd(gy, y, r):
    """Gradient of y = x * r(x): g_x = r * (g_y - y * mean(g_y * y))."""
    dot = np.mean(gy * y, axis=-1, keepdims=True, dtype=np.float64)
    return r * (gy - y * dot.astype(gy.dtype))


def rope_tables(T, D, theta):
    """cos and sin of phi[t, i] = t * theta^(-2i/D), i < D/2, in float64."""
    i = np.arange(D // 2, dtype=np.float64)
    inv = theta ** (-2.0 * i / D)
    phi = np.arange(T, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(phi), np.sin(phi)


def rope_fwd(x, cos, sin):
    """Rotate pairs (i, i + D/2) of x [B, T, heads, D] by +phi[t, i]."""
    h = x.shape[-1] // 2
    c = cos[None, :, None, :].astype(x.dtype)
    s = sin[None, :, None, :].astype(x.dtype)
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=-1)


def rope_bwd(g, cos, sin):
    """Transpose of the rotation = rotation by -phi."""
    h = g.shape[-1] // 2
    c = cos[None, :, None, :].astype(g.dtype)
    s = sin[None, :, None, :].astype(g.dtype)
    g1, g2 = g[..., :h], g[..., h:]
    return np.concatenate([g1 * c + g2 * s, -g1 * s + g2 * c], axis=-1)


def visible(T, full, W):
    """Boolean [T, T]: key s is visible to query t."""
    t = np.arange(T)[:, None]
    s = np.arange(T)[None, :]
    m = s <= t
    if not full:
        m &= (t - s) <= W
    return m


def _probs(qh, kh, mask, scale):
    S = np.matmul(qh, np.swapaxes(kh, -1, -2)) * qh.dtype.type(scale)
    S = np.where(mask, S, -np.inf)
    S -= S.max(axis=-1, keepdims=True)
    P = np.exp(S)
    P /= P.sum(axis=-1, keepdims=True, dtype=np.float64).astype(P.dtype)
    return P


def attention_fwd(q, k, v, full, W):
    """Causal (optionally windowed) GQA softmax attention, materialised.

    q [B, T, H, D]; k, v [B, T, Hk, D] -> y [B, T, H, D]."""
    B, T, H, D = q.shape
    Hk = k.shape[2]
    hmap = np.arange(H) // (H // Hk)
    mask = visible(T, full, W)
    y = np.empty_like(q)
    for b in range(B):
        qh = np.ascontiguousarray(q[b].transpose(1, 0, 2))
        kh = np.ascontiguousarray(k[b].transpose(1, 0, 2))[hmap]
        vh = np.ascontiguousarray(v[b].transpose(1, 0, 2))[hmap]
        P = _probs(qh, kh, mask, 1.0 / np.sqrt(D))
        y[b] = np.matmul(P, vh).transpose(1, 0, 2)
    return y


def attention_bwd(q, k, v, y, gy, full, W):
    """Gradients of attention_fwd: recompute P, then
    g_v = P^T g_y; g_P = g_y v^T; g_S = P (g_P - rowsum(g_y * y));
    g_q = g_S k / sqrt(D); g_k = g_S^T q / sqrt(D); K/V grads summed over
    the query heads that share them."""
    B, T, H, D = q.shape
    Hk = k.shape[2]
    G = H // Hk
    hmap = np.arange(H) // G
    mask = visible(T, full, W)
    scale = q.dtype.type(1.0 / np.sqrt(D))
    gq = np.empty_like(q)
    gk = np.zeros_like(k)
    gv = np.zeros_like(v)
    for b in range(B):
        qh = np.ascontiguousarray(q[b].transpose(1, 0, 2))
        kh = np.ascontiguousarray(k[b].transpose(1, 0, 2))[hmap]
        vh = np.ascontiguousarray(v[b].transpose(1, 0, 2))[hmap]
        yh = y[b].transpose(1, 0, 2)
        gyh = np.ascontiguousarray(gy[b].transpose(1, 0, 2))
        P = _probs(qh, kh, mask, 1.0 / np.sqrt(D))
        gvh = np.matmul(np.swapaxes(P, -1, -2), gyh)
        gP = np.matmul(gyh, np.swapaxes(vh, -1, -2))
        delta = np.sum(gyh * yh, axis=-1, keepdims=True, dtype=np.float64)
        gS = P * (gP - delta.astype(P.dtype))
        gq[b] = (np.matmul(gS, kh) * scale).transpose(1, 0, 2)
        gkh = np.matmul(np.swapaxes(gS, -1, -2), qh) * scale
        for h in range(H):
            gk[b, :, hmap[h]] += gkh[h]
            gv[b, :, hmap[h]] += gvh[h]
    return gq, gk, gv


def softcap_ce_fwd_bwd(z, targets, cap):
    """c = cap * tanh(z / cap); loss = mean over targets != -1 of
    logsumexp(c_n) - c_n[y_n]. Returns (loss as float64, g_z, c)."""
    c = cap * np.tanh(z / z.dtype.type(cap))
    m = c.max(axis=1, keepdims=True)
    e = np.exp(c - m)
    se = e.sum(axis=1, keepdims=True, dtype=np.float64)
    lse = m.astype(np.float64) + np.log(se)
    valid = targets >= 0
    n_valid = int(valid.sum())
    rows = np.nonzero(valid)[0]
    loss = float(np.sum(lse[rows, 0] - c[rows, targets[rows]].astype(np.float64))
                 / max(n_valid, 1))
    p = (e / se.astype(e.dtype))
    p[rows, targets[rows]] -= 1
    p[~valid] = 0
    gc = p / z.dtype.type(max(n_valid, 1))
    gz = gc * (1 - np.square(c / z.dtype.type(cap)))
    return loss, gz, c


# --------------------------------------------------------------------------
# Linear layers (optionally fp8-quantised, for the d26 configuration)
# --------------------------------------------------------------------------

class _Lin:
    """y = x W^T and its two gradients, plain or with per-tensor dynamic fp8
    ("additions" table: dynamic per-tensor fp8, e4m3 / e5m2; "overview"
    section 4: quantise and dequantise around each matmul). In fp8 mode the
    forward operands are quantised to e4m3 and the output gradient to e5m2,
    each with its own scale fmax / amax.

    fp8_round="bf16" rounds the activation and output-gradient operands to
    bfloat16 before they are quantised (weights are quantised from their
    fp32 values either way): the operands as a bf16-activation
    implementation holds them. Both variants are valid readings; the tests
    use the distance between them as the scale of fp8's own sensitivity."""

    def __init__(self, fp8: bool, fp8_round=None):
        self.fp8 = fp8
        assert fp8_round in (None, "bf16")
        self.rnd = (lambda a: _fp8.round_bf16(a).astype(a.dtype)) if fp8_round else (lambda a: a)

    def fwd(self, x, W):
        if self.fp8:
            x = _fp8.qdq(self.rnd(x), "e4m3")
            W = _fp8.qdq(W, "e4m3")
        return x @ W.T

    def bwd(self, gy, x, W):
        """(g_x, g_W)."""
        if self.fp8:
            gy = _fp8.qdq(self.rnd(gy), "e5m2")
            x = _fp8.qdq(self.rnd(x), "e4m3")
            W = _fp8.qdq(W, "e4m3")
        return gy @ W, gy.T @ x


def _sigmoid(a):
    return 1.0 / (1.0 + np.exp(-a))


def smear_fwd(e, w, B, T):
    """Smear ("additions" notes on Smear), readings as in the header:
    x0[b, t] = e[b, t] + sigmoid(e[b, t] . w) * e[b, t - 1] for t >= 1 and
    x0[b, 0] = e[b, 0]. e [B*T, C], w [1, C]. Returns x0 [B*T, C] and the
    gate values s [B, T] (s[:, 0] = 0: no gate there)."""
    C = e.shape[-1]
    e3 = e.reshape(B, T, C)
    s = np.zeros((B, T), dtype=e.dtype)
    s[:, 1:] = _sigmoid(e3[:, 1:] @ w.reshape(C))
    x0 = e3.copy()
    x0[:, 1:] += s[:, 1:, None] * e3[:, :-1]
    return x0.reshape(B * T, C), s


def smear_bwd(gx0, e, w, s, B, T):
    """Gradients of smear_fwd: (g_e [B*T, C], g_w [1, C]).
    Through x_prev: g_e[t - 1] += s[t] g[t]. Through the gate:
    dL/dz[t] = s[t] (1 - s[t]) <g[t], e[t - 1]>, z[t] = e[t] . w, so
    g_e[t] += dL/dz[t] w and g_w += dL/dz[t] e[t]."""
    C = e.shape[-1]
    g3 = gx0.reshape(B, T, C)
    e3 = e.reshape(B, T, C)
    ge = g3.copy()
    ge[:, :-1] += s[:, 1:, None] * g3[:, 1:]
    gs = np.sum(g3[:, 1:] * e3[:, :-1], axis=-1, dtype=np.float64).astype(e.dtype)
    gz = s[:, 1:] * (1 - s[:, 1:]) * gs
    ge[:, 1:] += gz[..., None] * w.reshape(1, 1, C)
    gw = gz.reshape(-1).astype(np.float64) @ e3[:, 1:].reshape(-1, C).astype(np.float64)
    return ge.reshape(B * T, C), gw.reshape(1, C)


def backout_layer(L: int) -> int:
    """Backout caches the residual stream entering this layer (the middle
    one; "additions" notes on Backout, reading in the header)."""
    return L // 2


# --------------------------------------------------------------------------
# The step
# --------------------------------------------------------------------------

def _layer_fwd(l, cfg, P, x, x0, tok, cos, sin, lin, dt):
    L = cfg.n_layer
    B, T = tok.shape
    N = B * T
    H, Hk, D = cfg.n_head, cfg.n_kv_head, cfg.head_dim
    eps = cfg.norm_eps
    c = {}
    lr = dt.type(P["resid_lambdas"][l])
    l0 = dt.type(P["x0_lambdas"][l])
    xin = lr * x + l0 * x0
    xn, r1 = rms_fwd(xin, eps)
    Wq, Wk, Wv = P[f"l{l}.q"].astype(dt), P[f"l{l}.k"].astype(dt), P[f"l{l}.v"].astype(dt)
    q = lin.fwd(xn, Wq).reshape(B, T, H, D)
    k = lin.fwd(xn, Wk).reshape(B, T, Hk, D)
    v = lin.fwd(xn, Wv).reshape(B, T, Hk, D)
    qn, rq = rms_fwd(rope_fwd(q, cos, sin), eps)
    kn, rk = rms_fwd(rope_fwd(k, cos, sin), eps)
    if layer_has_ve(l, L):
        Wg = P[f"l{l}.veg"].astype(dt)
        a = xn @ Wg.T                                    # [N, Hk]
        gate = _sigmoid(a)
        ve = P[f"l{l}.ve"].astype(dt)[tok.reshape(-1)].reshape(B, T, Hk, D)
        v = v + gate.reshape(B, T, Hk, 1) * ve
        c.update(a=a, gate=gate, ve=ve)
    full = layer_is_full(l, L)
    y = attention_fwd(qn, kn, v, full, cfg.short_window)
    Wo = P[f"l{l}.o"].astype(dt)
    xm = xin + lin.fwd(y.reshape(N, H * D), Wo)
    xn2, r2 = rms_fwd(xm, eps)
    u = lin.fwd(xn2, P[f"l{l}.fc"].astype(dt))
    h = np.square(np.maximum(u, 0))
    xo = xm + lin.fwd(h, P[f"l{l}.mp"].astype(dt))
    c.update(x=x, xin=xin, xn=xn, r1=r1, qn=qn, rq=rq, kn=kn, rk=rk, v=v, y=y,
             xm=xm, xn2=xn2, r2=r2, u=u, h=h, full=full)
    return xo, c


def _layer_bwd(l, cfg, P, c, gx, tok, cos, sin, lin, dt, G):
    """Backward of one block. gx: gradient w.r.t. the block output.
    Writes parameter grads into G; returns (g w.r.t. the block input x,
    g w.r.t. x0 from this block's mix)."""
    L = cfg.n_layer
    B, T = tok.shape
    N = B * T
    H, Hk, D = cfg.n_head, cfg.n_kv_head, cfg.head_dim
    # MLP: xo = xm + relu(u)^2 Wmp^T, u = xn2 Wfc^T
    Wfc, Wmp = P[f"l{l}.fc"].astype(dt), P[f"l{l}.mp"].astype(dt)
    gh, G[f"l{l}.mp"][...] = lin.bwd(gx, c["h"], Wmp)
    gu = gh * (2 * np.maximum(c["u"], 0))
    gxn2, G[f"l{l}.fc"][...] = lin.bwd(gu, c["xn2"], Wfc)
    gxm = gx + rms_bwd(gxn2, c["xn2"], c["r2"])
    # attention output projection: xm = xin + y Wo^T
    Wo = P[f"l{l}.o"].astype(dt)
    gy, G[f"l{l}.o"][...] = lin.bwd(gxm, c["y"].reshape(N, H * D), Wo)
    gxin = gxm.copy()
    gqn, gkn, gv = attention_bwd(c["qn"], c["kn"], c["v"], c["y"],
                                 gy.reshape(B, T, H, D), c["full"], cfg.short_window)
    Wq, Wk, Wv = P[f"l{l}.q"].astype(dt), P[f"l{l}.k"].astype(dt), P[f"l{l}.v"].astype(dt)
    xn = c["xn"]
    gxn = np.zeros_like(xn)
    if layer_has_ve(l, L):
        gate, ve = c["gate"], c["ve"]
        gve_rows = gate.reshape(B, T, Hk, 1) * gv                      # d ve
        ga = (gate * (1 - gate)) * np.sum(gv * ve, axis=-1, dtype=np.float64
                                          ).astype(dt).reshape(N, Hk)
        Wg = P[f"l{l}.veg"].astype(dt)
        G[f"l{l}.veg"][...] = (ga.astype(np.float64).T @ xn.astype(np.float64))
        gxn += ga @ Wg
        np.add.at(G[f"l{l}.ve"], tok.reshape(-1), gve_rows.reshape(N, Hk * D))
    gq = rope_bwd(rms_bwd(gqn, c["qn"], c["rq"]), cos, sin)
    gk = rope_bwd(rms_bwd(gkn, c["kn"], c["rk"]), cos, sin)
    for name, g, W in ((f"l{l}.q", gq, Wq), (f"l{l}.k", gk, Wk), (f"l{l}.v", gv, Wv)):
        gxi, G[name][...] = lin.bwd(g.reshape(N, -1), xn, W)
        gxn += gxi
    gxin += rms_bwd(gxn, xn, c["r1"])
    # mix: xin = lr * x + l0 * x0
    G["resid_lambdas"][l] = np.sum(gxin * c["x"], dtype=np.float64)
    G["x0_lambdas"][l] = np.sum(gxin * c["x0"], dtype=np.float64)
    lr = dt.type(P["resid_lambdas"][l])
    l0 = dt.type(P["x0_lambdas"][l])
    return lr * gxin, l0 * gxin


def forward_backward(cfg, params, tokens, targets, dtype=np.float64,
                     fp8=None, return_acts=False, fp8_round=None):
    """Loss and the flat gradient of every parameter, in canonical order.

    cfg: a workload description with the fields n_layer, n_embd, n_head,
    n_kv_head, head_dim, mlp_hidden, vocab, seq_len, batch, short_window,
    rope_theta, norm_eps, softcap, fp8_linears. params: flat fp32/fp64
    vector in the order of ``layout``. tokens, targets: int [B, T]; targets
    equal to -1 are ignored. dtype: array dtype of the computation.
    """
    dt = np.dtype(dtype)
    fp8 = cfg.fp8_linears if fp8 is None else fp8
    lin = _Lin(fp8, fp8_round)
    P = unpack(cfg, params)
    offs, total = param_offsets(cfg)
    grads = np.zeros(total, dtype=dt)
    G = unpack(cfg, grads)
    tok = np.asarray(tokens)
    tgt = np.asarray(targets).reshape(-1)
    B, T = tok.shape
    N = B * T
    L = cfg.n_layer
    cos, sin = rope_tables(T, cfg.head_dim, cfg.rope_theta)

    smear = getattr(cfg, "smear", False)
    backout = getattr(cfg, "backout", False)
    e = P["wte"].astype(dt)[tok.reshape(-1)]                   # [N, C]
    if smear:
        wsm = P["smear_gate"].astype(dt)
        x0, sg = smear_fwd(e, wsm, B, T)
    else:
        x0 = e
    xs = []
    x = x0
    acts = {}
    for l in range(L):
        xs.append(x)
        x, c = _layer_fwd(l, cfg, P, x, x0, tok, cos, sin, lin, dt)
        if return_acts:
            acts[l] = c
    mid = backout_layer(L)
    if backout:
        lb = dt.type(P["backout_lambda"][0])
        xb = x - lb * xs[mid]
    else:
        xb = x
    xf, rf = rms_fwd(xb, cfg.norm_eps)
    Wlm = P["lm_head"].astype(dt)
    z = xf @ Wlm.T
    loss, gz, cz = softcap_ce_fwd_bwd(z, tgt, cfg.softcap)
    if return_acts:
        acts["final"] = dict(x=x, xb=xb, xf=xf, rf=rf, c=cz, gz=gz, x0=x0)
    del z, cz
    G["lm_head"][...] = gz.T @ xf
    gx = rms_bwd(gz @ Wlm, xf, rf)               # w.r.t. the final norm input
    del gz
    if backout:
        G["backout_lambda"][0] = -np.sum(gx * xs[mid], dtype=np.float64)
        gbo = -lb * gx                            # joins the stream entering layer mid
    gx0 = np.zeros_like(x0)
    for l in reversed(range(L)):
        _, c = _layer_fwd(l, cfg, P, xs[l], x0, tok, cos, sin, lin, dt)
        c["x0"] = x0
        gx, g0 = _layer_bwd(l, cfg, P, c, gx, tok, cos, sin, lin, dt, G)
        gx0 += g0
        if backout and l == mid:
            gx = gx + gbo
        del c
    gx0 += gx                                     # layer 0 reads x = x0
    if smear:
        gx0, G["smear_gate"][...] = smear_bwd(gx0, e, wsm, sg, B, T)
    np.add.at(G["wte"], tok.reshape(-1), gx0)
    if return_acts:
        return loss, grads, acts
    return loss, grads


def forward_loss(cfg, params, tokens, targets, dtype=np.float64, fp8=None, fp8_round=None):
    """Loss only (the forward half of ``forward_backward``)."""
    dt = np.dtype(dtype)
    fp8 = cfg.fp8_linears if fp8 is None else fp8
    lin = _Lin(fp8, fp8_round)
    P = unpack(cfg, params)
    tok = np.asarray(tokens)
    B, T = tok.shape
    cos, sin = rope_tables(T, cfg.head_dim, cfg.rope_theta)
    x0 = P["wte"].astype(dt)[tok.reshape(-1)]
    if getattr(cfg, "smear", False):
        x0, _ = smear_fwd(x0, P["smear_gate"].astype(dt), B, T)
    x = x0
    xs = []
    for l in range(cfg.n_layer):
        xs.append(x)
        x, _ = _layer_fwd(l, cfg, P, x, x0, tok, cos, sin, lin, dt)
    if getattr(cfg, "backout", False):
        x = x - dt.type(P["backout_lambda"][0]) * xs[backout_layer(cfg.n_layer)]
    xf, _ = rms_fwd(x, cfg.norm_eps)
    z = xf @ P["lm_head"].astype(dt).T
    loss, _, _ = softcap_ce_fwd_bwd(z, np.asarray(targets).reshape(-1), cfg.softcap)
    return loss


def model_flops_per_token(cfg):
    """Model FLOPs per token, fwd + bwd: 6 per matrix weight used in a
    product plus 12 * H * D per visible key per layer (useful attention
    only). Test infrastructure mirror of the benchmark's accounting."""
    L, T, W = cfg.n_layer, cfg.seq_len, cfg.short_window
    n_mat = sum(int(np.prod(s)) for n, s in layout(cfg)
                if n.split(".")[-1] in ("q", "k", "v", "o", "fc", "mp", "veg")
                or n in ("lm_head", "smear_gate"))
    kbar = 0.0
    for l in range(L):
        if layer_is_full(l, L):
            kbar += (T + 1) / 2
        else:
            w = min(W, T - 1)
            kbar += (w * (w + 1) / 2 + (T - w) * (w + 1)) / T
    return 6 * n_mat + 12 * cfg.n_head * cfg.head_dim * kbar
