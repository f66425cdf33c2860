"""Seeded synthetic workloads for the attention path.

This module only draws random inputs; it holds none of the attention
arithmetic, so the tests can feed the same arrays to the HIP library and to
the CPU oracle.  Every array is drawn with numpy's PCG64 ``default_rng(seed)``
as float32 standard normals, scaled, and rounded to float16 once.

Draw order: the sequence lengths (variable-length workloads) or the boosted
key positions (long-context workload) first, then Q, K, V and dO.  V is drawn
as ``[B][KV][T][64]`` and handed over transposed, as the library's V^T
``[B][KV][64][T]``.

The five named workloads are the ones the path is measured and checked on;
the score scale is 1/sqrt(64) everywhere.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

HEAD_DIM = 64
SCALE = 1.0 / math.sqrt(HEAD_DIM)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    T: int
    heads: int
    kv_heads: int
    causal: bool
    seed: int
    varlen: bool = False        # lengths uniform in [1, T], padded to T
    qk_std: float = 1.0         # standard deviation of Q and K entries
    boost_frac: float = 0.0     # fraction of key rows per K/V head scaled by `boost`
    boost: float = 1.0


WORKLOADS = {
    "tiny_causal_t128": Workload("tiny_causal_t128", 1, 128, 1, 1, True, seed=1),
    "causal_mha_t1024": Workload("causal_mha_t1024", 1, 1024, 8, 8, True, seed=2),
    "causal_gqa_t4096": Workload("causal_gqa_t4096", 1, 4096, 32, 8, True, seed=3),
    "varlen_b16_t2048": Workload("varlen_b16_t2048", 16, 2048, 16, 16, False, seed=4, varlen=True),
    "long_causal_gqa_t16384": Workload("long_causal_gqa_t16384", 1, 16384, 32, 8, True, seed=5,
                                       qk_std=math.sqrt(2.0), boost_frac=0.01, boost=8.0),
}


def generate(w: Workload) -> dict:
    """Inputs of a workload: float16 Q, K, Vt, dO (numpy) and int32 seqlens or None."""
    return make_inputs(w.batch, w.T, w.heads, w.kv_heads, seed=w.seed, varlen=w.varlen,
                       qk_std=w.qk_std, boost_frac=w.boost_frac, boost=w.boost)


def make_inputs(batch, T, heads, kv_heads, *, seed, varlen=False, qk_std=1.0, boost_frac=0.0,
                boost=1.0, seqlens=None) -> dict:
    """Draw one problem's inputs.  `seqlens` may be given explicitly instead of drawn."""
    rng = np.random.default_rng(seed)
    if varlen and seqlens is None:
        seqlens = rng.integers(1, T + 1, size=batch).astype(np.int32)
    elif seqlens is not None:
        seqlens = np.asarray(seqlens, dtype=np.int32)
    boosted = None
    if boost_frac > 0.0:
        n = int(round(boost_frac * T))
        boosted = [[rng.choice(T, size=n, replace=False) for _ in range(kv_heads)] for _ in range(batch)]

    def normal(shape, std=1.0):
        x = rng.standard_normal(shape, dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        return x

    Q = normal((batch, heads, T, HEAD_DIM), qk_std).astype(np.float16)
    K = normal((batch, kv_heads, T, HEAD_DIM), qk_std)
    if boosted is not None:
        for b in range(batch):
            for kv in range(kv_heads):
                K[b, kv, boosted[b][kv], :] *= np.float32(boost)
    K = K.astype(np.float16)
    V = normal((batch, kv_heads, T, HEAD_DIM)).astype(np.float16)
    Vt = np.ascontiguousarray(V.transpose(0, 1, 3, 2))
    dO = normal((batch, heads, T, HEAD_DIM)).astype(np.float16)
    return {"Q": Q, "K": K, "Vt": Vt, "dO": dO, "seqlens": seqlens}
