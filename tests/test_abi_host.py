"""Host-side checks of the C ABI: the library loads, exports every function
include/gpt_step.h declares, validates configs, and reports the same
parameter layout and layer patterns as the oracle derives on its own.
Nothing here launches a kernel."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import workloads as W
from decoder_only_pretraining_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    txt = open(os.path.join(ROOT, "include", "gpt_step.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(gpt_[a-z_0-9]+)\s*\(", txt)))


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert "gpt_fwd_bwd" in names and len(names) >= 10
    lib = B.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(B.EXPORTS) == names


def test_abi_version():
    assert B.lib().gpt_abi_version() == B.GPT_ABI_VERSION


VARIANTS = {"tiny_smear": W.get("tiny").with_(smear=True),
            "tiny_backout": W.get("tiny").with_(backout=True),
            "d12_smear_backout": W.get("d12").with_(smear=True, backout=True)}


@pytest.mark.parametrize("name", list(W.CONFIGS) + list(VARIANTS))
def test_layout_matches_oracle(name):
    w = VARIANTS[name] if name in VARIANTS else W.get(name)
    cfg = B.make_config(w, fp8_linears=0)
    lay = B.param_layout(cfg)
    ref = [(n, o, s) for n, (o, s) in oracle.param_offsets(w)[0].items()]
    assert len(lay) == len(ref)
    for (n, o, r, c), (rn, ro, rs) in zip(lay, ref):
        assert n == rn and o == ro and (r * c) == int(np.prod(rs))
        assert (r, c) == (tuple(rs) if len(rs) == 2 else (rs[0], 1))
    assert B.param_count(cfg)[1] == oracle.param_offsets(w)[1]


@pytest.mark.parametrize("name", list(W.CONFIGS))
def test_layer_patterns_match_oracle(name):
    w = W.get(name)
    cfg = B.make_config(w, fp8_linears=0)
    for l in range(w.n_layer):
        assert B.layer_info(cfg, l) == (oracle.layer_is_full(l, w.n_layer),
                                        oracle.layer_has_ve(l, w.n_layer))


def test_validation_errors():
    w = W.get("tiny")
    ok = B.make_config(w)
    assert B.validate(ok) == 0
    bad = [dict(abi_version=7), dict(n_layer=0), dict(n_embd=100), dict(head_dim=96),
           dict(n_kv_head=3), dict(n_head=3, n_kv_head=2), dict(mlp_hidden=100),
           dict(vocab=500), dict(seq_len=0), dict(batch=0), dict(short_window=-1),
           dict(compute_dtype=5), dict(flags=256), dict(rope_theta=0.5), dict(norm_eps=0.0),
           dict(softcap=-1.0), dict(fp8_linears=2), dict(n_kv_head=32, n_head=32)]
    for kw in bad:
        assert B.validate(B.make_config(w, **kw)) == -1, kw
        assert B.lib().gpt_last_error().decode() != ""
    # fp8 linears run with bf16 compute only
    assert B.validate(B.make_config(w, fp8_linears=1)) == -1
    assert "bf16" in B.lib().gpt_last_error().decode()
    assert B.validate(B.make_config(w, fp8_linears=1, compute_dtype=B.GPT_DT_BF16)) == 0
    # the model-variant, debug and reuse flags are known bits
    assert B.validate(B.make_config(w, flags=B.GPT_F_SMEAR | B.GPT_F_BACKOUT | 1)) == 0
    assert B.validate(B.make_config(w, flags=B.GPT_F_CHECK_FINITE | B.GPT_F_CHECK_INPUTS |
                                    B.GPT_F_REUSE_WEIGHTS)) == 0
    # the embedding norm is a known bit that this library does not build
    assert B.validate(B.make_config(w, flags=B.GPT_F_EMBED_NORM)) == -5
    assert "EMBED_NORM" in B.lib().gpt_last_error().decode()
    assert B.lib().gpt_config_validate(None) == -2


def test_workspace_size_and_regions():
    w = W.get("d12")
    cfg = B.make_config(w)
    ws = B.workspace_size(cfg)
    N = w.batch * w.seq_len
    assert ws > N * w.vocab * 2      # holds the bf16 logits
    assert ws < 64 * 2 ** 30
    off, nb = B.workspace_region(cfg, "qkv", 3)
    assert nb == N * (w.n_head + 2 * w.n_kv_head) * w.head_dim * 2 and off % 256 == 0
    assert off + nb <= ws
    off, nb = B.workspace_region(cfg, "x", w.n_layer)
    assert nb == N * w.n_embd * 4 and off + nb <= ws
    with pytest.raises(B.GptError):
        B.workspace_region(cfg, "nope", 0)
    with pytest.raises(B.GptError):
        B.workspace_region(cfg, "xn", w.n_layer)


def test_entry_points_reject_bad_pointers_before_any_launch():
    w = W.get("tiny")
    cfg = B.make_config(w)
    L = B.lib()
    ws = B.workspace_size(cfg)
    p = ctypes.c_void_p(256)
    st = L.gpt_fwd_bwd(ctypes.byref(cfg), None, p, p, p, p, p, ws, None)
    assert st == -2
    st = L.gpt_fwd_bwd(ctypes.byref(cfg), ctypes.c_void_p(260), p, p, p, p, p, ws, None)
    assert st == -3
    st = L.gpt_fwd_bwd(ctypes.byref(cfg), p, p, p, p, p, p, ws - 1, None)
    assert st == -4
    st = L.gpt_fwd(ctypes.byref(cfg), p, p, p, p, p, ws - 1, None)
    assert st == -4
    cfg8 = B.make_config(w, fp8_linears=1)   # fp8 with fp32 compute
    assert L.gpt_fwd_bwd(ctypes.byref(cfg8), p, p, p, p, p, p, ws, None) == -1
    assert L.gpt_status_string(-4).decode() == "workspace too small"


GLOBAL_REGIONS = ["wc", "wct", "rope", "xin", "xf", "rf", "logits", "lossrow",
                  "scalars", "gx", "gxc", "gx0", "gu", "gtmp", "gO", "gqkv", "delta", "ga",
                  "lam_part", "veg_part", "vegrow", "tlink", "sgate", "part", "amax", "w8", "w8t", "q8", "g8t"]
LAYER_REGIONS = ["xn", "r1", "qkv", "rqk", "a", "attn", "lse", "xmid", "xn2", "r2", "h",
                 "x8t", "a8t", "x28t", "h8t"]


@pytest.mark.parametrize("name,fp8", [("tiny", 0), ("d12", 0), ("d12_gqa", 0), ("d26", 0),
                                      ("d26", 1), ("small_fp8", 1), ("d12_smear_backout", 0)])
def test_workspace_regions_disjoint(name, fp8):
    w = W.get(name) if name not in ("small_fp8", "d12_smear_backout") else W.get("d12").with_(
        n_layer=3, seq_len=200, batch=1, vocab=1024, fp8_linears=True)
    if name == "d12_smear_backout":
        w = VARIANTS[name]
    cfg = B.make_config(w, fp8_linears=fp8)
    ws = B.workspace_size(cfg)
    N, Np = w.batch * w.seq_len, (w.batch * w.seq_len + 127) // 128 * 128
    fp8_sizes = {"x8t": w.n_embd * Np, "a8t": w.n_head * w.head_dim * Np,
                 "x28t": w.n_embd * Np, "h8t": w.mlp_hidden * Np, "amax": 16 * w.n_layer * 4}
    for r, nb in fp8_sizes.items():
        assert B.workspace_region(cfg, r, 0)[1] == (nb if fp8 else 0), r
    spans = []
    for r in GLOBAL_REGIONS:
        spans.append((r, *B.workspace_region(cfg, r, 0)))
    for l in range(w.n_layer):
        for r in LAYER_REGIONS:
            spans.append((f"{r}[{l}]", *B.workspace_region(cfg, r, l)))
    for l in range(w.n_layer + 1):
        spans.append((f"x[{l}]", *B.workspace_region(cfg, "x", l)))
    spans = [s for s in spans if s[2] > 0]
    spans.sort(key=lambda s: s[1])
    for (n1, o1, b1), (n2, o2, b2) in zip(spans, spans[1:]):
        assert o1 + b1 <= o2, (n1, n2)
    assert all(o % 256 == 0 for _, o, _ in spans)
    N_sg = B.workspace_region(cfg, "sgate", 0)[1]
    assert N_sg == (4 * N if getattr(w, "smear", False) else 0)
    lam = B.workspace_region(cfg, "lam_part", 0)[1]
    slots = w.n_layer + (1 if getattr(w, "backout", False) else 0)
    assert lam >= slots * ((N + 3) // 4) * 2 * 4
    assert spans[-1][1] + spans[-1][2] <= ws


def test_fp8_quantize_rejects_bad_arguments_before_any_launch():
    L = B.lib()
    p = ctypes.c_void_p(4096)
    q = lambda *a: L.gpt_fp8_quantize(*a)
    assert q(None, 0, 4, 64, 0, p, p, 128, p, None) == -2            # src
    assert q(p, 0, 4, 64, 0, p, p, 128, None, None) == -2            # amax
    assert q(p, 7, 4, 64, 0, p, p, 128, p, None) == -1               # dtype
    assert q(p, 0, 4, 64, 3, p, p, 128, p, None) == -1               # format
    assert q(p, 0, 4, 96, 0, p, p, 128, p, None) == -1               # cols % 64
    assert q(p, 0, 0, 64, 0, p, p, 128, p, None) == -1               # rows
    assert q(p, 0, 200, 64, 0, p, p, 128, p, None) == -1             # pitch < rows
    assert q(p, 0, 4, 64, 0, p, p, 100, p, None) == -1               # pitch % 128
    assert q(ctypes.c_void_p(4100), 0, 4, 64, 0, p, p, 128, p, None) == -3
    assert q(p, 0, 4, 64, 0, ctypes.c_void_p(4104), None, 0, p, None) == -3


def test_bf16_gemm_rejects_bad_arguments_before_any_launch():
    L = B.lib()
    p = ctypes.c_void_p(4096)
    n = ctypes.c_size_t()
    g = L.gpt_bf16_gemm
    assert L.gpt_bf16_gemm_workspace(3, 64, 64, 64, ctypes.byref(n)) == -1   # kind
    assert L.gpt_bf16_gemm_workspace(0, 64, 96, 64, ctypes.byref(n)) == -1   # N % 64
    assert L.gpt_bf16_gemm_workspace(0, 64, 64, 32, ctypes.byref(n)) == -1   # K % 64
    assert L.gpt_bf16_gemm_workspace(2, 96, 64, 5, ctypes.byref(n)) == -1    # wgrad M % 64
    assert L.gpt_bf16_gemm_workspace(0, 64, 64, 64, None) == -2
    assert g(0, 64, 64, 64, None, p, 0, p, None, 0, None) == -2
    assert g(0, 64, 64, 64, p, p, 1, p, None, 0, None) == -1                 # accumulate, kind 0
    assert g(0, 64, 64, 64, ctypes.c_void_p(4100), p, 0, p, None, 0, None) == -3
    assert L.gpt_bf16_gemm_workspace(2, 3072, 768, 16384, ctypes.byref(n)) == 0 and n.value > 0
    assert g(2, 3072, 768, 16384, p, p, 0, p, p, n.value - 1, None) == -4


def test_fp8_gemm_k_segments_rejected_before_any_launch():
    """Scales along K (axis 2) are for the plain product only, with segment
    ends that are multiples of 16 within K; anything else returns
    GPT_E_INVAL before a launch (the pointers here are never dereferenced)."""
    L = B.lib()
    p = ctypes.c_void_p(1 << 20)
    g = L.gpt_fp8_gemm

    def sc(axis, ends, n):
        s = B.Fp8Scales()
        s.axis, s.nseg = axis, n
        for i, e in enumerate(ends):
            s.end[i] = e
        return s

    for wgrad, s in [(1, sc(2, [32], 2)), (0, sc(2, [40], 2)), (0, sc(2, [80], 2)),
                     (0, sc(2, [-16], 2)), (0, sc(2, [48, 32], 3)), (0, sc(3, [], 1))]:
        assert g(wgrad, 64, 64, 64, p, 64, 0, p, 64, p, ctypes.byref(s), 0, p, None, 0,
                 None) == -1, (wgrad, s.axis, list(s.end))


def test_decode_attn_validation_and_workspace():
    L = B.lib()
    # chunks of 128 visible positions per (sequence, KV head); one chunk: none
    assert B.decode_attn_workspace(16, 6, 6, 128, 2048, -1) == 16 * 6 * 16 * 130 * 4
    assert B.decode_attn_workspace(16, 6, 6, 128, 2048, 512) == 16 * 6 * 5 * 130 * 4
    assert B.decode_attn_workspace(2, 8, 2, 64, 3000, -1) == 2 * 8 * 24 * 66 * 4
    assert B.decode_attn_workspace(2, 4, 1, 64, 10, 0) == 0
    assert B.decode_attn_workspace(2, 4, 1, 64, 128, -1) == 0
    n = ctypes.c_size_t()
    for bad in [(0, 6, 6, 128, 64, -1), (2, 6, 4, 128, 64, -1), (2, 18, 2, 128, 64, -1),
                (2, 6, 6, 96, 64, -1), (2, 6, 6, 128, 0, -1), (2, 6, 6, 128, 64, -2)]:
        assert L.gpt_decode_attn_workspace(*bad, ctypes.byref(n)) == -1, bad
    p = ctypes.c_void_p(256)
    ws = B.decode_attn_workspace(2, 6, 6, 128, 1024, -1)
    assert ws > 0
    assert L.gpt_decode_attn(2, 6, 6, 128, 1024, -1, p, p, p, p, p, None, ws, None) == -2
    assert L.gpt_decode_attn(2, 6, 6, 128, 64, -1, None, p, p, p, p, p, ws, None) == -2
    assert L.gpt_decode_attn(2, 6, 6, 128, 64, -1, ctypes.c_void_p(264), p, p, p, p, p, ws,
                             None) == -3
    assert L.gpt_decode_attn(2, 6, 6, 128, 1024, -1, p, p, p, p, p, p, ws - 1, None) == -4


def test_optimizer_validation():
    w = W.get("tiny")
    cfg = B.make_config(w)
    L = B.lib()
    ws = B.optim_workspace_size(cfg)
    assert ws > 0
    p = ctypes.c_void_p(256)
    good = dict(step=1, ns_steps=5, nesterov=1, lr_matrix=0.02, lr_scalar=0.5, lr_embed=0.3,
                lr_unembed=0.008, lr_mult=1.0, weight_decay=0.28, beta1=0.9, beta2=0.999,
                eps=1e-8, momentum=0.95, ns_a=3.4445, ns_b=-4.775, ns_c=2.0315)
    for kw in [dict(step=0), dict(ns_steps=-1), dict(nesterov=2), dict(beta1=1.0),
               dict(beta2=-0.1), dict(lr_matrix=float("nan"))]:
        hp = B.OptimHparams(**dict(good, **kw))
        assert L.gpt_optimizer_step(ctypes.byref(cfg), ctypes.byref(hp), p, p, p, p, ws,
                                    None) == -1, kw
    hp = B.OptimHparams(**good)
    assert L.gpt_optimizer_step(ctypes.byref(cfg), ctypes.byref(hp), p, p, p, p, ws - 1,
                                None) == -4
    assert L.gpt_optimizer_step(ctypes.byref(cfg), ctypes.byref(hp), None, p, p, p, ws,
                                None) == -2
    assert L.gpt_optimizer_step(ctypes.byref(cfg), ctypes.byref(hp), ctypes.c_void_p(260), p, p,
                                p, ws, None) == -3


# ---------------------------------------------------------------- launch sequence
# Dry runs (gpt_debug_launches): the host logic of an entry point runs and
# counts its launches without launching anything, so none of these tests
# needs a GPU; fake device pointers are never dereferenced.

@pytest.fixture
def dry():
    B.debug_launches(-1, True)
    yield
    B.debug_launches(-1, False)


def _fake(n=7):
    return [ctypes.c_void_p(1 << 20) for _ in range(n)]


def _fwd_bwd(cfg):
    p = _fake()
    ws = B.workspace_size(cfg)
    return B.lib().gpt_fwd_bwd(ctypes.byref(cfg), p[0], p[1], p[2], p[3], p[4], p[5], ws, None)


def _fwd(cfg):
    p = _fake()
    ws = B.workspace_size(cfg)
    return B.lib().gpt_fwd(ctypes.byref(cfg), p[0], p[1], p[2], p[3], p[4], ws, None)


CASES = {"tiny": W.get("tiny"), "d12": W.get("d12"), "d12_gqa": W.get("d12_gqa"),
         "d26_fp8": W.get("d26"), "d12_smear_backout": VARIANTS["d12_smear_backout"]}


@pytest.mark.parametrize("name", list(CASES))
def test_dry_run_counts_the_launch_sequence(dry, name):
    cfg = B.make_config(CASES[name])
    assert _fwd_bwd(cfg) == 0
    n_step = B.debug_launch_count()
    assert _fwd_bwd(cfg) == 0 and B.debug_launch_count() == n_step   # deterministic
    assert _fwd(cfg) == 0
    n_fwd = B.debug_launch_count()
    assert 0 < n_fwd < n_step
    # the debug checks add their own launches: the id check (one), the
    # finiteness check (a flag clear and one pass over the loss, one over the
    # gradients in a backward call)
    assert _fwd_bwd(B.make_config(CASES[name], B.GPT_F_CHECK_INPUTS)) == 0
    assert B.debug_launch_count() == n_step + 1
    assert _fwd_bwd(B.make_config(CASES[name], B.GPT_F_CHECK_FINITE)) == 0
    assert B.debug_launch_count() == n_step + 3
    assert _fwd(B.make_config(CASES[name], B.GPT_F_CHECK_FINITE)) == 0
    assert B.debug_launch_count() == n_fwd + 2


@pytest.mark.parametrize("name", ["tiny", "d12", "d26_fp8"])
def test_injected_launch_failure_stops_the_sequence(name):
    cfg = B.make_config(CASES[name])
    B.debug_launches(-1, True)
    try:
        assert _fwd_bwd(cfg) == 0
        n_step = B.debug_launch_count()
        for k in sorted({0, 1, 7, n_step // 2, n_step - 1}):
            B.debug_launches(k, True)
            st = _fwd_bwd(cfg)
            assert st == -6, (k, st)                       # GPT_E_HIP
            assert B.debug_launch_count() == k             # nothing after the failed launch
            msg = B.lib().gpt_last_error().decode()
            assert "injected" in msg and f"launch {k}" in msg
        B.debug_launches(n_step, True)                     # past the last launch: no failure
        assert _fwd_bwd(cfg) == 0 and B.debug_launch_count() == n_step
        # the other entry points report it the same way
        B.debug_launches(0, True)
        p = _fake()
        assert B.lib().gpt_fp8_quantize(p[0], 1, 4, 64, 0, p[1], None, 0, p[2], None) == -6
        assert B.debug_launch_count() == 0
        ws = B.decode_attn_workspace(2, 6, 6, 128, 1024, -1)
        assert B.lib().gpt_decode_attn(2, 6, 6, 128, 1024, -1, p[0], p[1], p[2], p[3], p[4],
                                       p[5], ws, None) == -6
    finally:
        B.debug_launches(-1, False)
    assert B.lib().gpt_debug_launches(0, 2) == -1
