"""Decode attention over a KV cache (test infrastructure only).

The inference engine of the pages keeps a preallocated KV cache and, for
each generated token, attends the new token's queries to every cached
position ("Nanochat在nanoGPT之上的新增功能", section on the inference engine:
KV cache with pre-allocated tensors, batch-1 prefill then the cache copied
per sample; "nanochat — 架构与原理", section 5: the flash-attention call with
a KV cache). The attention itself is the model's: softmax(q k^T / sqrt(D))
over the visible keys, query head h reading KV head h // (H / Hk), and on
short-window layers only the keys at most `window` positions back (the
sliding-window notes of the additions page).

Plain definition: one query row per (sequence, head), scores, a softmax
with the maximum subtracted, the weighted sum of the value rows, in
float64.
"""
from __future__ import annotations

import numpy as np


def visible_range(t: int, window):
    """Cached positions s visible to the query at position t:
    max(0, t - window) <= s <= t (window None: 0 <= s <= t)."""
    lo = 0 if window is None or window < 0 else max(0, t - window)
    return lo, t + 1


def decode_attention(q, k, v, seqlen, window=None):
    """q [B, H, D]; k, v [B, Tmax, Hk, D]; seqlen [B] (the newest token of
    sequence b sits at position seqlen[b] - 1 and is already in the cache).
    Returns out [B, H, D] in float64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, D = q.shape
    Hk = k.shape[2]
    G = H // Hk
    out = np.zeros((B, H, D))
    for b in range(B):
        lo, hi = visible_range(int(seqlen[b]) - 1, window)
        for h in range(H):
            kk = k[b, lo:hi, h // G]                  # [n, D]
            vv = v[b, lo:hi, h // G]
            s = kk @ q[b, h] / np.sqrt(D)
            p = np.exp(s - s.max())
            out[b, h] = (p / p.sum()) @ vv
    return out


def kv_cache_append(qkv, pos, k_cache, v_cache, n_head, n_kv_head, head_dim):
    """Write the k and v rows of n_new tokens per sequence into the caches
    (in place): qkv [B * n_new, (H + 2 Hk) D] holds, per token, the q heads,
    then the k heads, then the v heads (the layout of the model's fused QKV
    product); token i of sequence b goes to position pos[b] + i. Positions
    outside the cache are not written."""
    H, Hk, D = n_head, n_kv_head, head_dim
    B, Tmax = k_cache.shape[:2]
    n_new = qkv.shape[0] // B
    for b in range(B):
        for i in range(n_new):
            p = int(pos[b]) + i
            if 0 <= p < Tmax:
                row = qkv[b * n_new + i]
                k_cache[b, p] = row[H * D:(H + Hk) * D].reshape(Hk, D)
                v_cache[b, p] = row[(H + Hk) * D:(H + 2 * Hk) * D].reshape(Hk, D)
