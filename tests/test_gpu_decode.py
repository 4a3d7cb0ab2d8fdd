"""Parity of the KV-cache decode attention (gpt_decode_attn) and the cache
append (gpt_kv_cache_append) with the CPU
oracle (oracle/decode.py) on seeded bf16 inputs.

Both sides read the same bf16 values; the oracle computes in float64. The
kernel accumulates in fp32 and rounds the result to bf16 once, so each
output element is within half a bf16 ulp of the exact value plus fp32
accumulation error: |out - ref| <= 2^-8 |ref| + 1e-4 elementwise (the
values are O(1)).

Shapes: the d12 attention (6 heads, head_dim 128) with 16 sequences (one
prompt's cache copied per sample) on a 2048-position cache, full-context
and 512-window layers; GQA 6:2 on a ragged 700-position cache; head_dim 64
with 8 query heads per KV head; one visible key (window 0, seqlen 1);
seqlen values outside [1, max_len], which the entry point clamps; few
(sequence, KV head) pairs with long caches, where the keys are split into
chunks and combined.
"""
import numpy as np
import pytest

import oracle
from decoder_only_pretraining_amd import binding as B

pytestmark = pytest.mark.gpu


def _bf16(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def _run(B_, H, Hk, D, Tmax, window, seqlen, seed):
    import torch
    rng = np.random.default_rng(seed)
    q = _bf16(rng.standard_normal((B_, H, D)))
    k = _bf16(rng.standard_normal((B_, Tmax, Hk, D)))
    v = _bf16(rng.standard_normal((B_, Tmax, Hk, D)))
    sl = torch.from_numpy(np.asarray(seqlen, dtype=np.int32))
    dev = "cuda"
    qd, kd, vd, sd = q.to(dev), k.to(dev), v.to(dev), sl.to(dev)
    out = torch.empty_like(qd)
    ws = torch.zeros(B.decode_attn_workspace(B_, H, Hk, D, Tmax, window), dtype=torch.uint8,
                     device=dev)
    B.decode_attn(qd, kd, vd, sd, out, ws, window)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    clamped = np.clip(np.asarray(seqlen), 1, Tmax)
    ref = oracle.decode.decode_attention(q.float().numpy(), k.float().numpy(), v.float().numpy(),
                                         clamped, None if window < 0 else window)
    return got, ref, (qd, kd, vd, sd, out, ws)


def _check(got, ref):
    err = np.abs(got - ref)
    bound = 2.0 ** -8 * np.abs(ref) + 1e-4
    assert np.all(err <= bound), (float(err.max()), np.unravel_index(np.argmax(err - bound), err.shape))


CASES = {
    "d12_full": (16, 6, 6, 128, 2048, -1),
    "d12_window": (16, 6, 6, 128, 2048, 512),
    "gqa_ragged": (5, 6, 2, 128, 700, 100),
    "d64_g8": (3, 8, 1, 64, 77, -1),
    "d64_window0": (3, 8, 2, 64, 77, 0),
    # few (sequence, KV head) pairs: the keys are split in chunks and combined
    "split_long": (1, 6, 6, 128, 8192, -1),
    "split_window": (1, 6, 6, 128, 8192, 1000),
    "split_gqa4_d64": (2, 8, 2, 64, 3000, -1),
    "split_g6": (2, 6, 1, 128, 2500, 700),
}


@pytest.mark.parametrize("name", list(CASES))
def test_decode_attention_parity(name):
    B_, H, Hk, D, Tmax, window = CASES[name]
    rng = np.random.default_rng(len(name))
    seqlen = rng.integers(1, Tmax + 1, B_)
    seqlen[0] = Tmax
    seqlen[-1] = 1
    got, ref, _ = _run(B_, H, Hk, D, Tmax, window, seqlen, seed=7 + len(name))
    _check(got, ref)


def test_decode_attention_clamps_seqlen_and_repeats_exactly():
    """Also: a second call on the same workspace gives the same bits."""
    import torch
    seqlen = [0, 5, 2000, -3]
    got, ref, (qd, kd, vd, sd, out, ws) = _run(4, 4, 2, 128, 1300, -1, seqlen, seed=3)
    _check(got, ref)
    first = out.clone()
    B.decode_attn(qd, kd, vd, sd, out, ws, -1)
    torch.cuda.synchronize()
    assert torch.equal(first, out)


def test_kv_cache_append_matches_oracle():
    """Bit-exact against the oracle's append, with positions that run past
    the cache end and one that starts before it."""
    import torch
    B_, n_new, H, Hk, D, Tmax = 3, 5, 6, 2, 128, 40
    rng = np.random.default_rng(11)
    qkv = _bf16(rng.standard_normal((B_ * n_new, (H + 2 * Hk) * D)))
    pos = np.array([0, 37, -2], dtype=np.int32)
    k0 = _bf16(rng.standard_normal((B_, Tmax, Hk, D)))
    v0 = _bf16(rng.standard_normal((B_, Tmax, Hk, D)))
    kd, vd = k0.cuda(), v0.cuda()
    B.kv_cache_append(qkv.cuda(), torch.from_numpy(pos).cuda(), kd, vd, H)
    torch.cuda.synchronize()
    kr, vr = k0.float().numpy(), v0.float().numpy()
    oracle.decode.kv_cache_append(qkv.float().numpy(), pos, kr, vr, H, Hk, D)
    np.testing.assert_array_equal(kd.float().cpu().numpy(), kr)
    np.testing.assert_array_equal(vd.float().cpu().numpy(), vr)


def test_prefill_then_decode_matches_the_forward_attention():
    """Prefill through the training forward: the per-layer qkv rows of a
    bf16 forward, appended to a cache, then decode attention for each
    sequence's last token, equal the forward's attention output at that
    token (both bf16; two roundings and different summation orders:
    |a - b| <= 2^-7 |b| + 2e-3), on a short-window and a full layer."""
    import torch
    import workloads as W
    from tests.gpu_common import inputs
    w = W.get("d12").with_(name="prefill", n_layer=4, seq_len=300, batch=3, short_window=75,
                           vocab=2048, n_kv_head=2)
    p, tok, tgt = inputs(w, 61, 62)
    step = B.Step(w, p, tok, tgt)
    step.forward()
    torch.cuda.synchronize()
    H, Hk, D, T, N = w.n_head, w.n_kv_head, w.head_dim, w.seq_len, w.batch * w.seq_len
    Tmax = T + 20
    for layer in (0, 3):                      # layer 0 short-window, layer 3 full
        window = -1 if oracle.layer_is_full(layer, w.n_layer) else w.short_window
        qkv = step.region("qkv", layer).view(torch.bfloat16).view(N, (H + 2 * Hk) * D)
        attn = step.region("attn", layer).view(torch.bfloat16).view(N, H * D)
        kc = torch.zeros(w.batch, Tmax, Hk, D, dtype=torch.bfloat16, device="cuda")
        vc = torch.zeros_like(kc)
        pos = torch.zeros(w.batch, dtype=torch.int32, device="cuda")
        B.kv_cache_append(qkv, pos, kc, vc, H)
        last = torch.arange(w.batch, device="cuda") * T + T - 1
        q = qkv[last, :H * D].reshape(w.batch, H, D).contiguous()
        out = torch.empty_like(q)
        ws = torch.empty(max(B.decode_attn_workspace(w.batch, H, Hk, D, Tmax, window), 1),
                         dtype=torch.uint8, device="cuda")
        seqlen = torch.full((w.batch,), T, dtype=torch.int32, device="cuda")
        B.decode_attn(q, kc, vc, seqlen, out, ws, window)
        torch.cuda.synchronize()
        got = out.float().cpu().numpy().reshape(w.batch, H * D)
        ref = attn[last].float().cpu().numpy()
        assert np.all(np.abs(got - ref) <= 2.0 ** -7 * np.abs(ref) + 2e-3), (
            layer, float(np.abs(got - ref).max()))
