"""Write the stored oracle results for the full-size workloads.

    python tests/golden/make_golden.py d12 d12_gqa d20 d26 [--variant-only]

For each workload: the oracle's loss, the full L2 norm of every gradient
tensor, and the sampled gradient entries chosen by sampling.py, from one
float32 oracle forward+backward on the seeded inputs. Calls only oracle/ and
workloads/.
"""
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))
sys.path.insert(0, HERE)

import oracle  # noqa: E402
import workloads as W  # noqa: E402
from sampling import sample_indices  # noqa: E402


def make(name, variant_only=False):
    """Stored results of one workload. For fp8 workloads also the oracle's
    fp8_round="bf16" variant (keys prefixed "r_"), the scale of fp8's own
    sensitivity used by the fp8 parity bar. variant_only: compute just that
    variant and merge it into the existing file."""
    w = W.get(name)
    offs, total = oracle.param_offsets(w)
    p = W.gen_params(total, w.n_layer, W.weight_seed(w))
    tok, tgt = W.split_tokens(W.gen_tokens(w))
    idx = sample_indices(offs, tok)
    path = os.path.join(HERE, f"{name}.npz")
    out = dict(np.load(path)) if variant_only else {}
    runs = [] if variant_only else [("", None)]
    if w.fp8_linears:
        runs.append(("r_", "bf16"))
    for prefix, rnd in runs:
        t0 = time.time()
        loss, g = oracle.forward_backward(w, p, tok, tgt, dtype=np.float32, fp8_round=rnd)
        dt = time.time() - t0
        out[prefix + "loss"] = np.float64(loss)
        out[prefix + "oracle_seconds"] = np.float64(dt)
        for k, (o, s) in offs.items():
            n = int(np.prod(s))
            out[prefix + "norm/" + k] = np.float64(np.linalg.norm(g[o:o + n].astype(np.float64)))
            out[prefix + "val/" + k] = g[o:o + n][idx[k]].astype(np.float32)
        del g
        print(f"{name}{' (' + prefix + ')' if prefix else ''}: loss {loss:.6f}, oracle {dt:.0f} s",
              flush=True)
    np.savez_compressed(path, **out)


if __name__ == "__main__":
    args = [a for a in sys.argv[1:] if not a.startswith("--")]
    for n in args:
        make(n, variant_only="--variant-only" in sys.argv)
