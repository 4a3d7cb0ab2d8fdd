"""Which gradient entries the stored full-size oracle results keep.

For every parameter tensor: all entries of the lambda vectors; for the
embedding tables (wte and the value-embedding tables) all columns of eight
rows that the batch uses (the four most frequent token ids and four drawn at
random among the others); for every other tensor 1024 entries drawn without
replacement. Indices are relative to the tensor's start and depend only on
the seed, the tensor's position and the batch's tokens.
"""
import numpy as np


def sample_indices(offsets, tokens, seed=4242, per_tensor=1024):
    """name -> int64 indices (relative to the tensor start)."""
    out = {}
    ids, counts = np.unique(np.asarray(tokens).reshape(-1), return_counts=True)
    order = ids[np.argsort(-counts, kind="stable")]
    for i, (name, (o, shape)) in enumerate(offsets.items()):
        rng = np.random.default_rng(seed + i)
        n = int(np.prod(shape))
        if name.endswith("lambdas"):
            idx = np.arange(n)
        elif name == "wte" or name.endswith(".ve"):
            rest = order[4:]
            pick = list(order[:4]) + list(rng.choice(rest, size=min(4, len(rest)), replace=False))
            cols = shape[1]
            idx = np.concatenate([np.arange(cols) + int(r) * cols for r in pick])
        else:
            idx = np.sort(rng.choice(n, size=min(per_tensor, n), replace=False))
        out[name] = idx.astype(np.int64)
    return out
