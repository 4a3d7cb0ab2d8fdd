"""ctypes binding of libgptstep.so (the gfx950 GPT step library).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/gpt_step.h. torch is used for
device memory and the current stream. The library must have been built
(``decoder_only_pretraining_amd.build``); loading fails loudly otherwise.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libgptstep.so")

GPT_ABI_VERSION = 2
GPT_DT_F32, GPT_DT_BF16 = 0, 1
GPT_F_ACCUMULATE = 1
GPT_F_EMBED_NORM = 2
GPT_F_CHECK_FINITE = 4
GPT_F_CHECK_INPUTS = 8
GPT_F_SMEAR = 16
GPT_F_BACKOUT = 32
GPT_F_REUSE_WEIGHTS = 64
GPT_F_GRAPH = 128

STATUS = {0: "GPT_OK", -1: "GPT_E_INVAL", -2: "GPT_E_NULLPTR", -3: "GPT_E_ALIGN",
          -4: "GPT_E_WORKSPACE", -5: "GPT_E_UNSUPPORTED", -6: "GPT_E_HIP",
          -7: "GPT_E_NONFINITE"}

EXPORTS = ["gpt_abi_version", "gpt_config_validate", "gpt_param_count", "gpt_param_info",
           "gpt_layer_info", "gpt_workspace_size", "gpt_workspace_region", "gpt_fwd_bwd",
           "gpt_fwd", "gpt_fp8_quantize", "gpt_status_string", "gpt_last_error",
           "gpt_profile_begin", "gpt_profile_end", "gpt_decode_attn_workspace",
           "gpt_decode_attn", "gpt_kv_cache_append", "gpt_optim_workspace_size",
           "gpt_optimizer_step", "gpt_debug_launches", "gpt_debug_launch_count",
           "gpt_decode_attn_noalloc", "gpt_attn_fwd", "gpt_attn_bwd", "gpt_fp8_gemm_workspace",
           "gpt_fp8_gemm", "gpt_graph_cache_clear", "gpt_bf16_gemm_workspace", "gpt_bf16_gemm"]
FP8_E4M3, FP8_E5M2 = 0, 1


class GptConfig(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_int32), ("n_layer", ctypes.c_int32),
                ("n_embd", ctypes.c_int32), ("n_head", ctypes.c_int32),
                ("n_kv_head", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("mlp_hidden", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("seq_len", ctypes.c_int32), ("batch", ctypes.c_int32),
                ("short_window", ctypes.c_int32), ("compute_dtype", ctypes.c_int32),
                ("fp8_linears", ctypes.c_int32), ("flags", ctypes.c_int32),
                ("rope_theta", ctypes.c_float), ("norm_eps", ctypes.c_float),
                ("softcap", ctypes.c_float)]


class Fp8Scales(ctypes.Structure):
    _fields_ = [("axis", ctypes.c_int32), ("nseg", ctypes.c_int32),
                ("end", ctypes.c_int64 * 2), ("slot_a", ctypes.c_int32 * 3),
                ("slot_b", ctypes.c_int32 * 3)]


class OptimHparams(ctypes.Structure):
    _fields_ = [("step", ctypes.c_int32), ("ns_steps", ctypes.c_int32),
                ("nesterov", ctypes.c_int32)] + [
        (n, ctypes.c_float) for n in ("lr_matrix", "lr_scalar", "lr_embed", "lr_unembed",
                                      "lr_mult", "weight_decay", "beta1", "beta2", "eps",
                                      "momentum", "ns_a", "ns_b", "ns_c")]


class GptError(RuntimeError):
    def __init__(self, fn, status, detail):
        super().__init__(f"{fn}: {STATUS.get(status, status)} ({detail})")
        self.status = status


_lib = None


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "python -m decoder_only_pretraining_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        c = ctypes
        P = c.POINTER
        L.gpt_abi_version.restype = c.c_int
        L.gpt_config_validate.argtypes = [P(GptConfig)]
        L.gpt_param_count.argtypes = [P(GptConfig), P(c.c_int64), P(c.c_int64)]
        L.gpt_param_info.argtypes = [P(GptConfig), c.c_int64, c.c_char_p, P(c.c_int64),
                                     P(c.c_int64), P(c.c_int64)]
        L.gpt_layer_info.argtypes = [P(GptConfig), c.c_int32, P(c.c_int32), P(c.c_int32)]
        L.gpt_workspace_size.argtypes = [P(GptConfig), P(c.c_size_t)]
        L.gpt_workspace_region.argtypes = [P(GptConfig), c.c_char_p, c.c_int32,
                                           P(c.c_size_t), P(c.c_size_t)]
        L.gpt_fwd_bwd.argtypes = [P(GptConfig), c.c_void_p, c.c_void_p, c.c_void_p, c.c_void_p,
                                  c.c_void_p, c.c_void_p, c.c_size_t, c.c_void_p]
        L.gpt_fwd.argtypes = [P(GptConfig), c.c_void_p, c.c_void_p, c.c_void_p, c.c_void_p,
                              c.c_void_p, c.c_size_t, c.c_void_p]
        L.gpt_fp8_quantize.argtypes = [c.c_void_p, c.c_int32, c.c_int64, c.c_int64, c.c_int32,
                                       c.c_void_p, c.c_void_p, c.c_int64, c.c_void_p, c.c_void_p]
        L.gpt_decode_attn_workspace.argtypes = [c.c_int32] * 6 + [P(c.c_size_t)]
        L.gpt_decode_attn.argtypes = [c.c_int32] * 6 + [c.c_void_p] * 6 + [c.c_size_t,
                                                                             c.c_void_p]
        L.gpt_kv_cache_append.argtypes = [c.c_int32] * 6 + [c.c_void_p] * 5
        L.gpt_decode_attn_noalloc.argtypes = [c.c_int32] * 6 + [c.c_void_p] * 6
        L.gpt_attn_fwd.argtypes = [P(GptConfig), c.c_int32] + [c.c_void_p] * 4
        L.gpt_attn_bwd.argtypes = [P(GptConfig), c.c_int32] + [c.c_void_p] * 7
        L.gpt_graph_cache_clear.argtypes = []
        L.gpt_fp8_gemm_workspace.argtypes = [c.c_int32, c.c_int64, c.c_int64, c.c_int64,
                                             P(c.c_size_t)]
        L.gpt_fp8_gemm.argtypes = [c.c_int32, c.c_int64, c.c_int64, c.c_int64, c.c_void_p,
                                   c.c_int64, c.c_int32, c.c_void_p, c.c_int64, c.c_void_p,
                                   P(Fp8Scales), c.c_int32, c.c_void_p, c.c_void_p, c.c_size_t,
                                   c.c_void_p]
        L.gpt_bf16_gemm_workspace.argtypes = [c.c_int32, c.c_int64, c.c_int64, c.c_int64,
                                              P(c.c_size_t)]
        L.gpt_bf16_gemm.argtypes = [c.c_int32, c.c_int64, c.c_int64, c.c_int64, c.c_void_p,
                                    c.c_void_p, c.c_int32, c.c_void_p, c.c_void_p, c.c_size_t,
                                    c.c_void_p]
        L.gpt_optim_workspace_size.argtypes = [P(GptConfig), P(c.c_size_t)]
        L.gpt_optimizer_step.argtypes = [P(GptConfig), P(OptimHparams)] + [c.c_void_p] * 4 + [
            c.c_size_t, c.c_void_p]
        L.gpt_debug_launches.argtypes = [c.c_int64, c.c_int32]
        L.gpt_debug_launch_count.argtypes = [P(c.c_int64)]
        L.gpt_status_string.restype = c.c_char_p
        L.gpt_status_string.argtypes = [c.c_int]
        L.gpt_last_error.restype = c.c_char_p
        L.gpt_profile_begin.argtypes = [c.c_char_p]
        L.gpt_profile_begin.restype = c.c_int
        L.gpt_profile_end.argtypes = [P(c.c_double), P(c.c_int64)]
        L.gpt_profile_end.restype = c.c_int
        for name in ("gpt_config_validate", "gpt_param_count", "gpt_param_info",
                     "gpt_layer_info", "gpt_workspace_size", "gpt_workspace_region",
                     "gpt_fwd_bwd", "gpt_fwd", "gpt_fp8_quantize", "gpt_decode_attn_workspace",
                     "gpt_decode_attn", "gpt_kv_cache_append", "gpt_optim_workspace_size",
                     "gpt_optimizer_step", "gpt_debug_launches", "gpt_debug_launch_count",
                     "gpt_decode_attn_noalloc", "gpt_attn_fwd", "gpt_attn_bwd",
                     "gpt_fp8_gemm_workspace", "gpt_fp8_gemm", "gpt_graph_cache_clear",
                     "gpt_bf16_gemm_workspace", "gpt_bf16_gemm"):
            getattr(L, name).restype = c.c_int
        if L.gpt_abi_version() != GPT_ABI_VERSION:
            raise RuntimeError("libgptstep.so ABI version mismatch")
        _lib = L
    return _lib


def _check(fn, st):
    if st != 0:
        raise GptError(fn, st, lib().gpt_last_error().decode())


def make_config(w, flags: int = 0, **over) -> GptConfig:
    """GptConfig from a workload description (attribute access). The model
    variant flags follow the description's ``smear`` / ``backout``."""
    if getattr(w, "smear", False):
        flags |= GPT_F_SMEAR
    if getattr(w, "backout", False):
        flags |= GPT_F_BACKOUT
    f = dict(abi_version=GPT_ABI_VERSION, n_layer=w.n_layer, n_embd=w.n_embd,
             n_head=w.n_head, n_kv_head=w.n_kv_head, head_dim=w.head_dim,
             mlp_hidden=w.mlp_hidden, vocab=w.vocab, seq_len=w.seq_len, batch=w.batch,
             short_window=w.short_window,
             compute_dtype=GPT_DT_BF16 if w.compute_dtype == "bf16" else GPT_DT_F32,
             fp8_linears=int(bool(w.fp8_linears)), flags=flags, rope_theta=w.rope_theta,
             norm_eps=w.norm_eps, softcap=w.softcap)
    f.update(over)
    return GptConfig(**f)


def validate(cfg: GptConfig) -> int:
    return lib().gpt_config_validate(ctypes.byref(cfg))


def param_count(cfg):
    nt, ne = ctypes.c_int64(), ctypes.c_int64()
    _check("gpt_param_count", lib().gpt_param_count(ctypes.byref(cfg), ctypes.byref(nt),
                                                    ctypes.byref(ne)))
    return nt.value, ne.value


def param_layout(cfg):
    """[(name, offset, rows, cols)] in canonical order."""
    nt, _ = param_count(cfg)
    out = []
    buf = ctypes.create_string_buffer(64)
    o, r, c = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    for i in range(nt):
        _check("gpt_param_info", lib().gpt_param_info(ctypes.byref(cfg), i, buf, ctypes.byref(o),
                                                      ctypes.byref(r), ctypes.byref(c)))
        out.append((buf.value.decode(), o.value, r.value, c.value))
    return out


def layer_info(cfg, l):
    f, v = ctypes.c_int32(), ctypes.c_int32()
    _check("gpt_layer_info", lib().gpt_layer_info(ctypes.byref(cfg), l, ctypes.byref(f),
                                                  ctypes.byref(v)))
    return bool(f.value), bool(v.value)


def workspace_size(cfg) -> int:
    b = ctypes.c_size_t()
    _check("gpt_workspace_size", lib().gpt_workspace_size(ctypes.byref(cfg), ctypes.byref(b)))
    return b.value


def workspace_region(cfg, name: str, layer: int = 0):
    o, b = ctypes.c_size_t(), ctypes.c_size_t()
    _check("gpt_workspace_region", lib().gpt_workspace_region(
        ctypes.byref(cfg), name.encode(), layer, ctypes.byref(o), ctypes.byref(b)))
    return o.value, b.value


def _stream_ptr(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def fwd_bwd(cfg, params, tokens, targets, loss, grads, workspace, stream=None):
    """Enqueue one forward+backward on `stream` (default: torch's current
    stream). All tensors are device tensors owned by the caller."""
    st = lib().gpt_fwd_bwd(ctypes.byref(cfg), params.data_ptr(), tokens.data_ptr(),
                           targets.data_ptr(), loss.data_ptr(), grads.data_ptr(),
                           workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                           _stream_ptr(stream))
    _check("gpt_fwd_bwd", st)


def fwd(cfg, params, tokens, targets, loss, workspace, stream=None):
    st = lib().gpt_fwd(ctypes.byref(cfg), params.data_ptr(), tokens.data_ptr(),
                       targets.data_ptr(), loss.data_ptr(), workspace.data_ptr(),
                       workspace.numel() * workspace.element_size(), _stream_ptr(stream))
    _check("gpt_fwd", st)


def attn_fwd(cfg, full, qkv, out, lse2, stream=None):
    """gpt_attn_fwd on device tensors: qkv [N, (H + 2 Hk) D], out [N, H D]
    (compute dtype), lse2 fp32 of B H T + 64 elements."""
    st = lib().gpt_attn_fwd(ctypes.byref(cfg), int(full), qkv.data_ptr(), out.data_ptr(),
                            lse2.data_ptr(), _stream_ptr(stream))
    _check("gpt_attn_fwd", st)


def attn_bwd(cfg, full, qkv, out, g_out, lse2, delta, g_qkv, stream=None):
    """gpt_attn_bwd on device tensors (delta: fp32 scratch like lse2)."""
    st = lib().gpt_attn_bwd(ctypes.byref(cfg), int(full), qkv.data_ptr(), out.data_ptr(),
                            g_out.data_ptr(), lse2.data_ptr(), delta.data_ptr(), g_qkv.data_ptr(),
                            _stream_ptr(stream))
    _check("gpt_attn_bwd", st)


def fp8_quantize(src, fmt, codes=None, codes_t=None, pitch_t=0, amax=None, stream=None):
    """Per-tensor fp8 codes of the 2-D device tensor `src` (fp32 or bf16):
    row-major into `codes` and/or transposed into `codes_t` [cols, pitch_t]
    (uint8 device tensors), the bit pattern of max |src| into `amax`
    (int32 device tensor of one element)."""
    import torch
    rows, cols = src.shape
    dt = GPT_DT_BF16 if src.dtype == torch.bfloat16 else GPT_DT_F32
    ptr = lambda t: None if t is None else t.data_ptr()
    st = lib().gpt_fp8_quantize(src.data_ptr(), dt, rows, cols, fmt, ptr(codes), ptr(codes_t),
                                pitch_t, ptr(amax), _stream_ptr(stream))
    _check("gpt_fp8_quantize", st)


def fp8_gemm(wgrad, A, lda, fmt_a, B, ldb, amax, scales, C, M, N, K, accumulate=False,
             stream=None):
    """gpt_fp8_gemm on device tensors (A, B uint8 codes, amax int32 slots, C
    fp32 [M, N]); allocates the weight-gradient partials itself."""
    import torch
    n = ctypes.c_size_t()
    _check("gpt_fp8_gemm_workspace", lib().gpt_fp8_gemm_workspace(int(wgrad), M, N, K,
                                                                  ctypes.byref(n)))
    ws = torch.empty(max(n.value, 1), dtype=torch.uint8, device=C.device)
    st = lib().gpt_fp8_gemm(int(wgrad), M, N, K, A.data_ptr(), lda, fmt_a, B.data_ptr(), ldb,
                            amax.data_ptr(), ctypes.byref(scales), int(accumulate), C.data_ptr(),
                            ws.data_ptr(), n.value, _stream_ptr(stream))
    _check("gpt_fp8_gemm", st)
    return ws


GEMM_NT, GEMM_NT_SPLITK, GEMM_WGRAD = 0, 1, 2


def bf16_gemm(kind, A, B, C, M, N, K, accumulate=False, stream=None):
    """gpt_bf16_gemm on device tensors (A, B bf16, C fp32 [M, N]); allocates
    the split-K partials itself and returns them."""
    import torch
    n = ctypes.c_size_t()
    _check("gpt_bf16_gemm_workspace", lib().gpt_bf16_gemm_workspace(kind, M, N, K,
                                                                    ctypes.byref(n)))
    ws = torch.empty(max(n.value, 1), dtype=torch.uint8, device=C.device)
    st = lib().gpt_bf16_gemm(kind, M, N, K, A.data_ptr(), B.data_ptr(), int(accumulate),
                             C.data_ptr(), ws.data_ptr(), n.value, _stream_ptr(stream))
    _check("gpt_bf16_gemm", st)
    return ws


def decode_attn_workspace(batch, n_head, n_kv_head, head_dim, max_len, window) -> int:
    n = ctypes.c_size_t()
    _check("gpt_decode_attn_workspace",
           lib().gpt_decode_attn_workspace(batch, n_head, n_kv_head, head_dim, max_len, window,
                                           ctypes.byref(n)))
    return n.value


def decode_attn(q, k_cache, v_cache, seqlen, out, workspace, window=-1, stream=None):
    """Decode attention (gpt_decode_attn) on device tensors: q, out bf16
    [B, H, D]; caches bf16 [B, Tmax, Hk, D]; seqlen int32 [B]; workspace a
    device tensor of at least decode_attn_workspace(...) bytes."""
    B, H, D = q.shape
    _, Tmax, Hk, _ = k_cache.shape
    st = lib().gpt_decode_attn(B, H, Hk, D, Tmax, window, q.data_ptr(), k_cache.data_ptr(),
                               v_cache.data_ptr(), seqlen.data_ptr(), out.data_ptr(),
                               workspace.data_ptr(),
                               workspace.numel() * workspace.element_size(), _stream_ptr(stream))
    _check("gpt_decode_attn", st)


def decode_attn_noalloc(q, k_cache, v_cache, seqlen, out, window=-1, stream=None):
    """gpt_decode_attn_noalloc: decode_attn with the library's static scratch
    instead of a workspace (for callers that cannot allocate)."""
    B, H, D = q.shape
    _, Tmax, Hk, _ = k_cache.shape
    st = lib().gpt_decode_attn_noalloc(B, H, Hk, D, Tmax, window, q.data_ptr(),
                                       k_cache.data_ptr(), v_cache.data_ptr(), seqlen.data_ptr(),
                                       out.data_ptr(), _stream_ptr(stream))
    _check("gpt_decode_attn_noalloc", st)


def kv_cache_append(qkv, pos, k_cache, v_cache, n_head, stream=None):
    """gpt_kv_cache_append on device tensors: qkv bf16 [B * n_new, (H + 2 Hk) D],
    pos int32 [B], caches bf16 [B, Tmax, Hk, D]."""
    B, Tmax, Hk, D = k_cache.shape
    n_new = qkv.shape[0] // B
    st = lib().gpt_kv_cache_append(B, n_new, n_head, Hk, D, Tmax, qkv.data_ptr(), pos.data_ptr(),
                                   k_cache.data_ptr(), v_cache.data_ptr(), _stream_ptr(stream))
    _check("gpt_kv_cache_append", st)


def optim_workspace_size(cfg) -> int:
    n = ctypes.c_size_t()
    _check("gpt_optim_workspace_size", lib().gpt_optim_workspace_size(ctypes.byref(cfg),
                                                                      ctypes.byref(n)))
    return n.value


def optimizer_step(cfg, hp: OptimHparams, params, grads, state, workspace, stream=None):
    """gpt_optimizer_step on device tensors (fp32 params, grads, state [2 n];
    workspace uint8)."""
    st = lib().gpt_optimizer_step(ctypes.byref(cfg), ctypes.byref(hp), params.data_ptr(),
                                  grads.data_ptr(), state.data_ptr(), workspace.data_ptr(),
                                  workspace.numel() * workspace.element_size(),
                                  _stream_ptr(stream))
    _check("gpt_optimizer_step", st)


def debug_launches(fail_at: int = -1, dry_run: bool = False):
    """Fault injection / dry run of the calling thread's later calls
    (gpt_debug_launches): launch number `fail_at` fails (< 0: none);
    dry_run counts the launch sequence without launching."""
    _check("gpt_debug_launches", lib().gpt_debug_launches(fail_at, 1 if dry_run else 0))


def debug_launch_count() -> int:
    """Launches issued (or counted) by the thread's last entry-point call."""
    n = ctypes.c_int64()
    _check("gpt_debug_launch_count", lib().gpt_debug_launch_count(ctypes.byref(n)))
    return n.value


def profile_begin(site_prefix: str):
    _check("gpt_profile_begin", lib().gpt_profile_begin(site_prefix.encode()))


def profile_end():
    """(summed kernel milliseconds, launches) since profile_begin."""
    ms, n = ctypes.c_double(), ctypes.c_int64()
    _check("gpt_profile_end", lib().gpt_profile_end(ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


class Step:
    """Device buffers for repeated calls on one workload: params, grads,
    tokens, targets, loss and the workspace, allocated once with torch."""

    def __init__(self, w, params_np, tokens_np, targets_np, flags=0, device="cuda"):
        import torch
        self.cfg = make_config(w, flags)
        _check("gpt_config_validate", validate(self.cfg))
        self.n_tensors, self.n_elems = param_count(self.cfg)
        assert params_np.size == self.n_elems
        self.params = torch.from_numpy(params_np).to(device)
        self.grads = torch.empty(self.n_elems, dtype=torch.float32, device=device)
        self.tokens = torch.from_numpy(tokens_np).to(device).contiguous()
        self.targets = torch.from_numpy(targets_np).to(device).contiguous()
        self.loss = torch.zeros(1, dtype=torch.float32, device=device)
        self.ws_bytes = workspace_size(self.cfg)
        self.workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)

    def run(self, stream=None):
        fwd_bwd(self.cfg, self.params, self.tokens, self.targets, self.loss, self.grads,
                self.workspace, stream)

    def forward(self, stream=None):
        fwd(self.cfg, self.params, self.tokens, self.targets, self.loss, self.workspace, stream)

    def region(self, name, layer=0):
        """A saved forward tensor inside the workspace (see gpt_workspace_region)."""
        import torch
        off, nbytes = workspace_region(self.cfg, name, layer)
        return self.workspace[off:off + nbytes]
