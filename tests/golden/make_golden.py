"""Write the stored oracle results for the full-size workloads.

    python tests/golden/make_golden.py d12 d12_gqa d20

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


def make(name):
    w = W.get(name)
    offs, total = oracle.param_offsets(w)
    p = W.gen_params(total, w.n_layer, W.weight_seed(w))
    tok, tgt = W.split_tokens(W.gen_tokens(w))
    t0 = time.time()
    loss, g = oracle.forward_backward(w, p, tok, tgt, dtype=np.float32)
    dt = time.time() - t0
    idx = sample_indices(offs, tok)
    out = {"loss": np.float64(loss), "oracle_seconds": np.float64(dt)}
    for k, (o, s) in offs.items():
        n = int(np.prod(s))
        out["norm/" + k] = np.float64(np.linalg.norm(g[o:o + n].astype(np.float64)))
        out["val/" + k] = g[o:o + n][idx[k]].astype(np.float32)
    np.savez_compressed(os.path.join(HERE, f"{name}.npz"), **out)
    print(f"{name}: loss {loss:.6f}, oracle {dt:.0f} s", flush=True)


if __name__ == "__main__":
    for n in sys.argv[1:]:
        make(n)
