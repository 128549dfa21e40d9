"""Seeded generators.  Inputs only: nothing here computes any part of the method.

Seeding: ``np.random.SeedSequence(seed).spawn(h)`` gives one child per head; each
head's child is spawned again into three streams (keys, values, queries), each
drawn with ``np.random.default_rng``.  Keys of a head are drawn as one (n, d)
block, so a smaller n yields a prefix of the same stream for the per-vector
distributions (sphere, gauss_clip); gauss_rescale rescales by the set's own
maximum norm, so it is prefix-stable only up to that single factor.
"""

import numpy as np

from .configs import Workload


def vectors(rng: np.random.Generator, count: int, d: int, dist: str,
            r: float) -> np.ndarray:
    """``count`` vectors in R^d drawn in float64 and returned as float32."""
    g = rng.standard_normal((count, d))
    if dist == "sphere":
        nrm = np.linalg.norm(g, axis=1, keepdims=True)
        x = r * g / nrm
    elif dist == "gauss_rescale":
        nrm = np.linalg.norm(g, axis=1)
        x = g * (r / nrm.max()) if count else g
    elif dist == "gauss_clip":
        nrm = np.linalg.norm(g, axis=1, keepdims=True)
        x = g * np.minimum(1.0, r / nrm)
    else:
        raise ValueError(f"unknown vector distribution {dist!r}")
    return np.ascontiguousarray(x, dtype=np.float32)


def values(rng: np.random.Generator, count: int, dv: int, dist: str) -> np.ndarray:
    if dist == "uniform":
        x = rng.uniform(-1.0, 1.0, (count, dv))
    elif dist == "normal":
        x = rng.standard_normal((count, dv))
    else:
        raise ValueError(f"unknown value distribution {dist!r}")
    return np.ascontiguousarray(x, dtype=np.float32)


def _head_rngs(seed: int, h: int):
    for child in np.random.SeedSequence(seed).spawn(h):
        kk, vv, qq = child.spawn(3)
        yield (np.random.default_rng(kk), np.random.default_rng(vv),
               np.random.default_rng(qq))


def generate_head(w: Workload, head: int):
    """(K, V, Q) of one head: float32 arrays [n, d], [n, dv], [m, d]."""
    if not 0 <= head < w.h:
        raise IndexError(head)
    for i, (rk, rv, rq) in enumerate(_head_rngs(w.seed, w.h)):
        if i == head:
            K = vectors(rk, w.n, w.d, w.key_dist, w.key_r)
            V = values(rv, w.n, w.dv, w.val_dist)
            Q = vectors(rq, w.m, w.d, w.key_dist, w.key_r)
            return K, V, Q
    raise AssertionError("unreachable")


def generate(w: Workload):
    """(K, V, Q) for all heads: float32 arrays [h, n, d], [h, n, dv], [h, m, d]."""
    K = np.empty((w.h, w.n, w.d), np.float32)
    V = np.empty((w.h, w.n, w.dv), np.float32)
    Q = np.empty((w.h, w.m, w.d), np.float32)
    for i, (rk, rv, rq) in enumerate(_head_rngs(w.seed, w.h)):
        K[i] = vectors(rk, w.n, w.d, w.key_dist, w.key_r)
        V[i] = values(rv, w.n, w.dv, w.val_dist)
        Q[i] = vectors(rq, w.m, w.d, w.key_dist, w.key_r)
    return K, V, Q
