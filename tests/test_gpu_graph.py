"""GPT_F_GRAPH: the call's launch sequence captured once into a HIP graph and
replayed. Every replay must equal the eager call on the same inputs (bit
for bit, except the embedding tables, whose fp32 atomic sums may differ in
order: relative L2 1e-6), with eager work on the GPU and host
synchronisations between the replays; a change of the buffers' contents
(not of the pointers) between replays must show in the next replay. Also:
the null stream and the debug checks are refused with GPT_F_GRAPH."""
import ctypes

import numpy as np
import pytest

import oracle
import workloads as W
from decoder_only_pretraining_amd import binding as B
from tests.gpu_common import inputs, per_tensor

pytestmark = pytest.mark.gpu

SMALL = W.get("d12").with_(name="small_bf16", n_layer=4, seq_len=300, batch=2,
                           short_window=75, vocab=2048)


def _same(w, g, ref, what):
    offs = oracle.param_offsets(w)[0]
    for name, (o, shp) in offs.items():
        n = int(np.prod(shp))
        if name == "wte" or name.endswith(".ve"):
            assert per_tensor(w, g, ref)[name][0] <= 1e-6, (what, name)
        else:
            assert np.array_equal(g[o:o + n], ref[o:o + n]), (what, name)


@pytest.mark.parametrize("w", [W.get("tiny"), SMALL], ids=lambda w: w.name)
def test_graph_replays_equal_eager(w):
    import torch
    p, tok, tgt = inputs(w, 81, 82)
    step = B.Step(w, p, tok, tgt)
    torch.cuda.synchronize()                          # uploads on the default stream done
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        step.run(s)                                   # eager reference
        s.synchronize()
        l_ref, g_ref = float(step.loss.item()), step.grads.cpu().numpy().copy()
        gcfg = B.make_config(w, B.GPT_F_GRAPH)
        for i in range(4):
            step.grads.fill_(float("nan"))
            step.loss.fill_(float("nan"))
            B.fwd_bwd(gcfg, step.params, step.tokens, step.targets, step.loss, step.grads,
                      step.workspace, s)              # i = 0 captures, then replays
            s.synchronize()
            assert float(step.loss.item()) == l_ref, i
            _same(w, step.grads.cpu().numpy(), g_ref, f"replay {i}")
            # eager work between replays: the eager call itself, and torch ops
            step.run(s)
            torch.matmul(torch.ones(64, 64, device="cuda"), torch.ones(64, 64, device="cuda"))
            s.synchronize()
        # new contents behind the same pointers: the replay sees them
        offs = oracle.param_offsets(w)[0]
        o, shp = offs["lm_head"]
        step.params[o:o + int(np.prod(shp))] *= 2.0
        step.run(s)
        s.synchronize()
        l2, g2 = float(step.loss.item()), step.grads.cpu().numpy().copy()
        assert l2 != l_ref
        B.fwd_bwd(gcfg, step.params, step.tokens, step.targets, step.loss, step.grads,
                  step.workspace, s)
        s.synchronize()
        assert float(step.loss.item()) == l2
        _same(w, step.grads.cpu().numpy(), g2, "after the parameter change")
        # the forward-only call has its own graph
        step.loss.fill_(0.0)
        B.fwd(gcfg, step.params, step.tokens, step.targets, step.loss, step.workspace, s)
        s.synchronize()
        assert float(step.loss.item()) == l2
    assert B.lib().gpt_graph_cache_clear() == 0


def test_graph_flag_rules():
    import torch
    w = W.get("tiny")
    p, tok, tgt = inputs(w)
    step = B.Step(w, p, tok, tgt)
    L = B.lib()
    for flags, stream in [(B.GPT_F_GRAPH, None),
                          (B.GPT_F_GRAPH | B.GPT_F_CHECK_FINITE, torch.cuda.Stream()),
                          (B.GPT_F_GRAPH | B.GPT_F_CHECK_INPUTS, torch.cuda.Stream())]:
        cfg = B.make_config(w, flags)
        sp = None if stream is None else ctypes.c_void_p(stream.cuda_stream)
        st = L.gpt_fwd_bwd(ctypes.byref(cfg), step.params.data_ptr(), step.tokens.data_ptr(),
                           step.targets.data_ptr(), step.loss.data_ptr(), step.grads.data_ptr(),
                           step.workspace.data_ptr(), step.ws_bytes, sp)
        assert st == -1, (flags, st)
        assert "GPT_F_GRAPH" in L.gpt_last_error().decode()
