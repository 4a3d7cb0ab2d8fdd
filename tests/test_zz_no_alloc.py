"""gpt_decode_attn_noalloc (the decode attention entry point for callers that
cannot allocate: its chunk states live in the library's static scratch)
against gpt_decode_attn with a caller workspace, through the C ABI: two
calls in a row, the second smaller, each equal to the workspace entry
point's output bit for bit (same kernels, same inputs) and within the
decode tolerance of the oracle (|out - ref| <= 2^-8 |ref| + 1e-4, the
bound of tests/test_gpu_decode.py); sizes past the scratch are refused."""
import ctypes

import numpy as np
import pytest

import oracle
from decoder_only_pretraining_amd import binding as B

pytestmark = pytest.mark.gpu


def _bf16(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def _inputs(B_, H, Hk, D, Tmax, seqlen, seed):
    import torch
    rng = np.random.default_rng(seed)
    q = _bf16(rng.standard_normal((B_, H, D)))
    k = _bf16(rng.standard_normal((B_, Tmax, Hk, D)))
    v = _bf16(rng.standard_normal((B_, Tmax, Hk, D)))
    sl = torch.from_numpy(np.asarray(seqlen, dtype=np.int32))
    return q, k, v, sl


def test_noalloc_equals_workspace_entry_point_twice_second_smaller():
    import torch
    rng = np.random.default_rng(31)
    cases = [
        # d12 decode shape: 16 sequences x 6 heads x 16 chunks of full context
        (16, 6, 6, 128, 2048, -1, rng.integers(1, 2049, 16).tolist() + []),
        # smaller: GQA 8:2, head_dim 64, a 300-key window over a ragged cache
        (3, 8, 2, 64, 700, 300, [700, 1, 455]),
    ]
    cases[0][6][0] = 2048
    results = []
    for B_, H, Hk, D, Tmax, window, seqlen in cases:
        q, k, v, sl = _inputs(B_, H, Hk, D, Tmax, seqlen, 100 + B_)
        qd, kd, vd, sd = (t.to("cuda") for t in (q, k, v, sl))
        out_na = torch.full_like(qd, float("nan"))
        st = B.lib().gpt_decode_attn_noalloc(B_, H, Hk, D, Tmax, window, qd.data_ptr(),
                                             kd.data_ptr(), vd.data_ptr(), sd.data_ptr(),
                                             out_na.data_ptr(),
                                             ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert st == 0, B.lib().gpt_last_error()
        torch.cuda.synchronize()
        results.append((B_, H, Hk, D, Tmax, window, seqlen, q, k, v, sl, qd, kd, vd, sd,
                        out_na.clone()))
    for (B_, H, Hk, D, Tmax, window, seqlen, q, k, v, sl, qd, kd, vd, sd, out_na) in results:
        out_ws = torch.full_like(qd, float("nan"))
        ws = torch.zeros(B.decode_attn_workspace(B_, H, Hk, D, Tmax, window), dtype=torch.uint8,
                         device="cuda")
        B.decode_attn(qd, kd, vd, sd, out_ws, ws, window)
        torch.cuda.synchronize()
        assert torch.equal(out_na.view(torch.int16), out_ws.view(torch.int16))
        got = out_na.float().cpu().numpy()
        ref = oracle.decode.decode_attention(q.float().numpy(), k.float().numpy(),
                                             v.float().numpy(), np.asarray(seqlen),
                                             None if window < 0 else window)
        err = np.abs(got - ref)
        assert np.all(err <= 2.0 ** -8 * np.abs(ref) + 1e-4), float(err.max())


def test_noalloc_refuses_sizes_past_the_scratch():
    import torch
    # 64 sequences x 16 heads x 16 chunks x 130 floats = 8.5 MB > 4 MiB
    assert B.decode_attn_workspace(64, 16, 16, 128, 2048, -1) > 4 << 20
    p = torch.zeros(16, dtype=torch.uint8, device="cuda")
    ptr = p.data_ptr()
    st = B.lib().gpt_decode_attn_noalloc(64, 16, 16, 128, 2048, -1, ptr, ptr, ptr, ptr, ptr, None)
    assert st == -4
    assert "static scratch" in B.lib().gpt_last_error().decode()
    # the largest d12 decode that fits: 8065 chunk states of head_dim 128
    assert B.decode_attn_workspace(84, 6, 6, 128, 2048, -1) <= 4 << 20 < \
        B.decode_attn_workspace(85, 6, 6, 128, 2048, -1)
