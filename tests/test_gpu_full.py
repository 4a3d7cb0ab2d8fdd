"""Full-size workloads (the launch configuration bench.py times) against the
oracle's stored results: the loss, and every parameter tensor's gradient on
the entries chosen by tests/golden/sampling.py (all of them for the lambda
vectors, eight used rows of each embedding table, 1024 seeded entries of
every other tensor). The stored values come from
tests/golden/make_golden.py, which calls only the oracle.

Bar (bf16): loss relative error <= 1e-2; per-tensor cosine >= 0.999 on the
sampled entries; the full gradient norm within 5% of the oracle's.
fp8 linears (d26): loss relative error <= 1e-2; per tensor, the relative L2
error on the sampled entries within tests/gpu_common.fp8_bounds of the
distance between the stored oracle results and the stored results of its
bf16-rounding variant (fp8 codes are discontinuous in their inputs), and
the full gradient norm within 5% of the oracle's for the partially sampled
tensors (for the lambda vectors, sampled whole, the relative L2 bound is
the stronger statement: it bounds |norm ratio - 1| by itself).
"""
import os

import numpy as np
import pytest

import oracle
import workloads as W
from tests.golden.sampling import sample_indices
from tests.gpu_common import fp8_bounds, gpu_step, inputs

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


@pytest.mark.parametrize("name", ["d12", "d12_gqa", "d20", "d26"])
def test_full_size_against_stored_oracle(name):
    path = os.path.join(GOLDEN, f"{name}.npz")
    if not os.path.exists(path):
        pytest.skip(f"no stored oracle results for {name}")
    ref = np.load(path)
    w = W.get(name)
    if w.fp8_linears and "r_loss" not in ref:
        pytest.skip(f"stored results for {name} lack the fp8 bf16-rounding variant")
    p, tok, tgt = inputs(w)
    lg, gg, _ = gpu_step(w, p, tok, tgt)
    lo = float(ref["loss"])
    assert abs(lg - lo) <= 1e-2 * abs(lo), (lg, lo)
    offs, _ = oracle.param_offsets(w)
    idx = sample_indices(offs, tok)
    if w.fp8_linears:
        bound = fp8_bounds(w, {k: _rel(ref["r_val/" + k].astype(np.float64),
                                       ref["val/" + k].astype(np.float64)) for k in offs})
    bad = {}
    for k, (o, s) in offs.items():
        n = int(np.prod(s))
        full = gg[o:o + n].astype(np.float64)
        a = full[idx[k]]
        b = ref["val/" + k].astype(np.float64)
        ratio = float(np.linalg.norm(full) / ref["norm/" + k])
        if w.fp8_linears:
            # where the sample is the whole tensor (the lambda vectors) its
            # rel-L2 bound already bounds the norm ratio (|ratio - 1| <=
            # rel L2); the 5% norm check covers the partially sampled ones
            whole = idx[k].size == n
            ok = _rel(a, b) <= bound[k] and (whole or abs(ratio - 1) <= 0.05)
            if not ok:
                bad[k] = (_rel(a, b), bound[k], ratio)
        else:
            cos = float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))
            if not (cos >= 0.999 and abs(ratio - 1) <= 0.05):
                bad[k] = (cos, ratio)
    assert not bad, bad
