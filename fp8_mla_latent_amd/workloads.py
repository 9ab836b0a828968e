"""Seeded synthetic inputs for the fp8 latent-KV MLA decode workloads.

This module only draws numbers: it holds none of the method's arithmetic (no
encoding, no scaling, no attention), so the HIP path and the CPU oracle can both
consume what it produces.  All draws use numpy's PCG64 with a fixed seed.

The shapes follow the workloads of colibri PR #300 ("KV8 long-context CUDA:
fp8 device shadow, split-T kernels, DSA-aware gather"): absorbed MLA decode in
the DeepSeek-V3 regime (kv_lora 512, qk_rope 64) over a long fp8 latent cache,
the selected-row (DSA) gather decode, and the batched causal path.  The pages
measure on real models; standard-normal rows and queries stand in for them.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    n_heads: int
    lc: int
    rc: int
    t_rows: int          # rows attended (after any append)
    seed: int
    sm_scale: float
    n_sel: int = 0       # selected rows (gather decode)
    n_q: int = 0         # query positions (batched causal)
    n_append: int = 1    # fresh rows quantized and appended before attention
    outlier_frac: float = 0.0
    outlier_mult: float = 1.0

    @property
    def d(self) -> int:
        return self.lc + self.rc


# sm_scale = 1/sqrt(qk_nope_head_dim + qk_rope_head_dim) of the model family:
# 1/sqrt(64 + 16) for the tiny shape, 1/sqrt(128 + 64) for DeepSeek-V3 shapes.
TINY = Workload("tiny", 4, 64, 16, 256, seed=1, sm_scale=1.0 / math.sqrt(80.0))
DSV3 = Workload("dsv3_t4096", 128, 512, 64, 4096, seed=2, sm_scale=1.0 / math.sqrt(192.0),
                outlier_frac=0.01, outlier_mult=50.0)
LONG = Workload("long_t262144", 64, 512, 64, 262144, seed=3, sm_scale=1.0 / math.sqrt(192.0))
DSA = Workload("dsa_t131072_ns2048", 64, 512, 64, 131072, seed=4,
               sm_scale=1.0 / math.sqrt(192.0), n_sel=2048)
BATCH = Workload("batch_s64_t32768", 64, 512, 64, 32768, seed=5,
                 sm_scale=1.0 / math.sqrt(192.0), n_q=64, n_append=64)

# fp8 indexer over the DSA shadow's rows: 64 indexer heads of dimension 128
# (n_heads = n_ih, lc = ihd), one 128-byte e4m3 key row per cached row,
# top-k = the gather's 2048 rows.
DSA_INDEX = Workload("dsa_index_t131072_k2048", 64, 128, 0, 131072, seed=6, sm_scale=1.0,
                     n_sel=2048)

ALL = {w.name: w for w in (TINY, DSV3, LONG, DSA, BATCH, DSA_INDEX)}


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def rows(w: Workload, n: int, seed_offset: int = 0) -> np.ndarray:
    """f32 latent rows [n, Lc+Rc] ~ N(0,1); a seeded fraction of whole rows is
    multiplied by ``outlier_mult`` (outlier amax) when the workload asks for it."""
    g = rng(w.seed * 1000 + seed_offset)
    x = g.standard_normal((n, w.d), dtype=np.float32)
    if w.outlier_frac > 0.0:
        k = int(round(w.outlier_frac * n))
        idx = g.choice(n, size=k, replace=False)
        x[idx] *= np.float32(w.outlier_mult)
    return x


def queries(w: Workload, seed_offset: int = 0) -> tuple[np.ndarray, np.ndarray]:
    """(q_lat, q_rope) f32 ~ N(0,1): [H, Lc], [H, Rc], or [S, H, *] for a batch."""
    g = rng(w.seed * 1000 + 500 + seed_offset)
    lead = (w.n_q, w.n_heads) if w.n_q else (w.n_heads,)
    q_lat = g.standard_normal(lead + (w.lc,), dtype=np.float32)
    q_rope = g.standard_normal(lead + (w.rc,), dtype=np.float32)
    return q_lat, q_rope


def selection(w: Workload, t_rows: int | None = None, seed_offset: int = 0) -> np.ndarray:
    """``n_sel`` sorted unique absolute row indices, uniform over [0, t_rows)."""
    t = w.t_rows if t_rows is None else t_rows
    g = rng(w.seed * 1000 + 700 + seed_offset)
    return np.sort(g.choice(t, size=w.n_sel, replace=False)).astype(np.int32)


def index_weights(w: Workload, seed_offset: int = 0) -> np.ndarray:
    """Indexer head weights [n_ih] f32 ~ N(0, 1/n_ih) (either sign)."""
    g = rng(w.seed * 1000 + 900 + seed_offset)
    return (g.standard_normal(w.n_heads) / np.sqrt(w.n_heads)).astype(np.float32)
