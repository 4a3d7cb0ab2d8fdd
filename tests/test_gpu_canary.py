"""Canary words around and between the buffers of a call: the forward+
backward writes only the gradients, the loss and the workspace regions that
gpt_workspace_region lists. Every caller buffer gets a guard tail filled
with a byte pattern, the workspace is filled with the pattern before the
call, and after the call the guard tails, the alignment gaps between the
listed workspace regions, and the read-only inputs (parameters, tokens,
targets) must be unchanged. Workloads: the fp32 config, a ragged bf16
config, the d12 widths at seq 2048 with GQA, the Smear / Backout variants and
the fp8 linears."""
import numpy as np
import pytest

import workloads as W
from decoder_only_pretraining_amd import binding as B
from tests.gpu_common import inputs
from tests.test_abi_host import GLOBAL_REGIONS, LAYER_REGIONS

pytestmark = pytest.mark.gpu

GUARD = 1 << 16  # bytes of canary after each buffer
PAT = 0xA5

CASES = {
    "tiny_fp32": W.get("tiny"),
    "ragged_bf16": W.get("d12").with_(name="ragged", n_layer=2, seq_len=77, batch=3,
                                      vocab=640),
    "d12w_gqa_t2048": W.get("d12").with_(name="d12w_gqa", n_layer=4, batch=1, n_kv_head=2),
    "smear_backout": W.get("d12").with_(name="sb", n_layer=4, seq_len=150, batch=2, vocab=2048,
                                        smear=True, backout=True),
    "fp8": W.get("d12").with_(name="f8", n_layer=3, seq_len=200, batch=1, vocab=1024,
                              fp8_linears=True),
}


def _guarded(nbytes, device="cuda"):
    """A uint8 buffer of nbytes + GUARD filled with the pattern, and the
    view of its first nbytes."""
    import torch
    buf = torch.full((nbytes + GUARD,), PAT, dtype=torch.uint8, device=device)
    return buf, buf[:nbytes]


def _gaps(cfg, w, ws):
    spans = []
    for r in GLOBAL_REGIONS:
        spans.append(B.workspace_region(cfg, r, 0))
    for l in range(w.n_layer):
        for r in LAYER_REGIONS:
            spans.append(B.workspace_region(cfg, r, l))
    for l in range(w.n_layer + 1):
        spans.append(B.workspace_region(cfg, "x", l))
    spans = sorted(s for s in spans if s[1] > 0)
    gaps, end = [], 0
    for o, n in spans:
        if o > end:
            gaps.append((end, o))
        end = max(end, o + n)
    gaps.append((end, ws))
    return [(a, b) for a, b in gaps if b > a]


@pytest.mark.parametrize("name", sorted(CASES))
def test_call_writes_only_its_outputs_and_regions(name):
    import torch
    w = CASES[name]
    cfg = B.make_config(w)
    params_np, tok, tgt = inputs(w)
    tok = np.ascontiguousarray(tok, dtype=np.int32)
    tgt = np.ascontiguousarray(tgt, dtype=np.int32)
    params_np = np.ascontiguousarray(params_np, dtype=np.float32)
    n = params_np.size
    ws = B.workspace_size(cfg)

    pbuf, pview = _guarded(4 * n)
    pview.copy_(torch.from_numpy(params_np.view(np.uint8)).cuda())
    gbuf, gview = _guarded(4 * n)
    tbuf, tview = _guarded(tok.nbytes)
    tview.copy_(torch.from_numpy(tok.view(np.uint8).reshape(-1)).cuda())
    ybuf, yview = _guarded(tgt.nbytes)
    yview.copy_(torch.from_numpy(tgt.view(np.uint8).reshape(-1)).cuda())
    lbuf, lview = _guarded(4)
    wbuf, wview = _guarded(ws)
    before = {k: v.clone() for k, v in (("params", pbuf), ("tokens", tbuf), ("targets", ybuf))}
    torch.cuda.synchronize()

    B.fwd_bwd(cfg, pview.view(torch.float32), tview.view(torch.int32), yview.view(torch.int32),
              lview.view(torch.float32), gview.view(torch.float32), wview)
    torch.cuda.synchronize()

    for k, buf in (("params", pbuf), ("tokens", tbuf), ("targets", ybuf)):
        assert torch.equal(buf, before[k]), f"{k} (or its guard) changed"
    for k, buf, nb in (("grads", gbuf, 4 * n), ("loss", lbuf, 4), ("workspace", wbuf, ws)):
        tail = buf[nb:].cpu().numpy()
        assert np.all(tail == PAT), (k, "guard overwritten at byte", int(np.argmax(tail != PAT)))
    host = wbuf[:ws].cpu().numpy()
    for a, b in _gaps(cfg, w, ws):
        bad = np.nonzero(host[a:b] != PAT)[0]
        assert bad.size == 0, ("workspace gap", a, b, "written at", int(a + bad[0]))
    assert np.isfinite(lview.view(torch.float32).item())
    assert bool(torch.isfinite(gview.view(torch.float32)).all())
