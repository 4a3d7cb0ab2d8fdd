"""Seeded synthetic workloads: model configurations and input generators.

This module is shared by the CPU oracle, the tests and the benchmark. It
holds no part of the model's arithmetic: it only describes workload sizes
and draws seeded random numbers (weights, token streams).

The configurations follow the nanochat d12 training report ("NanoChat基础训练
报告", model architecture block) for d12, and the depth dial of the nanochat
architecture overview (section 4: width = depth x 64, head_dim 128) for d20
and d26. The token stream stands in for the FineWeb-Edu / ClimbMix text the
pages train on: a bounded Zipf(1.1) draw over the 32,768-id vocabulary
(the vocabulary size of the d12 report), which has the heavy head of a real
BPE token stream.
"""
from __future__ import annotations

from dataclasses import dataclass, asdict, replace
import numpy as np

__all__ = ["Workload", "CONFIGS", "get", "gen_params", "gen_tokens",
           "split_tokens", "zipf_tokens"]


@dataclass(frozen=True)
class Workload:
    name: str
    n_layer: int
    n_embd: int
    n_head: int
    n_kv_head: int
    head_dim: int
    mlp_hidden: int
    vocab: int
    seq_len: int
    batch: int
    short_window: int
    compute_dtype: str          # "f32" | "bf16"
    fp8_linears: bool
    seed_index: int             # k in the seed rules below
    token_dist: str             # "uniform" | "zipf"
    rope_theta: float = 10000.0
    norm_eps: float = 2.0 ** -23
    softcap: float = 15.0
    # model variants of the nanochat additions page (notes on Smear and
    # Backout); off in the configurations below
    smear: bool = False
    backout: bool = False

    @property
    def tokens_per_call(self) -> int:
        return self.batch * self.seq_len

    def as_dict(self):
        return asdict(self)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


CONFIGS = {
    "tiny": Workload("tiny", 2, 128, 2, 2, 64, 512, 512, 64, 2, 16,
                     "f32", False, 0, "uniform"),
    "d12": Workload("d12", 12, 768, 6, 6, 128, 3072, 32768, 2048, 8, 512,
                    "bf16", False, 1, "zipf"),
    "d12_gqa": Workload("d12_gqa", 12, 768, 6, 2, 128, 3072, 32768, 2048, 16,
                        512, "bf16", False, 2, "zipf"),
    "d20": Workload("d20", 20, 1280, 10, 10, 128, 5120, 32768, 2048, 16, 512,
                    "bf16", False, 3, "zipf"),
    "d26": Workload("d26", 26, 1664, 13, 13, 128, 6656, 32768, 2048, 8, 512,
                    "bf16", True, 4, "zipf"),
}


def get(name: str) -> Workload:
    return CONFIGS[name]


def gen_params(n_total: int, n_layer: int, seed: int,
               std: float = 0.02, lam_resid: float = 1.0,
               lam_x0: float = 0.1) -> np.ndarray:
    """Flat fp32 parameter vector.

    Every entry is drawn N(0, std^2) from ``numpy.random.default_rng(seed)``
    in one pass; the last ``2*n_layer`` entries (the per-layer residual and
    x0 mixing scalars, which close the canonical layout) are then set to
    ``lam_resid`` and ``lam_x0``. The caller supplies the total size.
    """
    rng = np.random.default_rng(seed)
    p = rng.standard_normal(n_total, dtype=np.float32)
    p *= np.float32(std)
    p[n_total - 2 * n_layer:n_total - n_layer] = lam_resid
    p[n_total - n_layer:] = lam_x0
    return p


def zipf_tokens(shape, vocab: int, s: float, rng) -> np.ndarray:
    """Bounded Zipf(s) ids by inverse CDF: rank r in 1..vocab has mass
    proportional to r^-s; the id is r - 1."""
    ranks = np.arange(1, vocab + 1, dtype=np.float64)
    cdf = np.cumsum(ranks ** (-s))
    cdf /= cdf[-1]
    u = rng.random(shape)
    ids = np.searchsorted(cdf, u, side="right")
    return np.minimum(ids, vocab - 1).astype(np.int32)


def gen_tokens(w: Workload, seed: int | None = None) -> np.ndarray:
    """int32 [batch, seq_len + 1] stream; inputs are [:, :T], targets [:, 1:]."""
    rng = np.random.default_rng(2000 + w.seed_index if seed is None else seed)
    shape = (w.batch, w.seq_len + 1)
    if w.token_dist == "uniform":
        return rng.integers(0, w.vocab, shape).astype(np.int32)
    return zipf_tokens(shape, w.vocab, 1.1, rng)


def split_tokens(stream: np.ndarray):
    """(tokens, targets), both C-contiguous int32 [B, T]."""
    return (np.ascontiguousarray(stream[:, :-1]),
            np.ascontiguousarray(stream[:, 1:]))


def weight_seed(w: Workload) -> int:
    return 1000 + w.seed_index
