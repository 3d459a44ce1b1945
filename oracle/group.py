"""V-Smooth Group: k-means grouping of the value tokens of one head and the
joint permutation of keys and values.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: VC-Attention article (aikraft.ru), section 02, Group: an online
k-means clusters the value tokens of each batch and head; keys and values are
permuted together, so non-causal attention output is unchanged; grouping runs
on the first quarter of the denoising steps and a permutation is reused for
four neighbouring steps; after sorting, subtracting the mean of each 128-token
block removes far more of the block's energy (36%) than in sequence order (8%).

Readings taken where the article is silent: Lloyd's k-means with a fixed
number of rounds on the 128 channels of each V token (the article names only
"online k-means"); ``n_clusters`` defaults to ceil(S / 128), one cluster per
hardware block on average; deterministic start: centroid c is token floor(c
* S / n_clusters); assignment: argmin over c of |mu_c|^2 - 2 v . mu_c (the
token's own norm is the same for every c), ties to the lowest c; update: the
mean of the assigned tokens, an empty cluster keeps its centroid; after the
last update one more assignment; the permutation lists the tokens by
(cluster, token index), i.e. a stable sort by cluster. "Energy removed" by
block means is sum_b n_b |mean_b|^2 / sum_j |v_j|^2 (what subtracting each
block's mean takes out of the sum of squares). """

from __future__ import annotations

import numpy as np

from .attention import _as_f64

__all__ = [
    "initial_centroids",
    "assign",
    "update",
    "kmeans_head",
    "stable_permutation",
    "objective",
    "block_energy_removed",
]


def initial_centroids(v, n_clusters: int) -> np.ndarray:
    """Centroid c = token floor(c * S / n_clusters)."""
    v = _as_f64(v)
    S = v.shape[0]
    idx = (np.arange(n_clusters, dtype=np.int64) * S) // n_clusters
    return v[idx].copy()


def assign(v, centroids, block: int = 4096) -> np.ndarray:
    """Nearest centroid of every token: argmin_c |mu_c|^2 - 2 v . mu_c,
    ties to the lowest index (numpy's argmin)."""
    v = _as_f64(v)
    mu = np.asarray(centroids, np.float64)
    m2 = (mu * mu).sum(axis=1)
    out = np.empty(v.shape[0], np.int64)
    for r0 in range(0, v.shape[0], block):
        d = m2[None, :] - 2.0 * (v[r0:r0 + block] @ mu.T)
        out[r0:r0 + block] = np.argmin(d, axis=1)
    return out


def update(v, labels, centroids) -> np.ndarray:
    """Mean of each cluster's tokens; an empty cluster keeps its centroid."""
    v = _as_f64(v)
    k = centroids.shape[0]
    sums = np.zeros_like(centroids, dtype=np.float64)
    np.add.at(sums, labels, v)
    counts = np.bincount(labels, minlength=k)
    new = np.array(centroids, np.float64, copy=True)
    nz = counts > 0
    new[nz] = sums[nz] / counts[nz, None]
    return new


def kmeans_head(v, n_clusters: int | None = None, rounds: int = 4):
    """Lloyd's k-means on the value tokens of one head [S, D]: ``rounds``
    (assign, update) rounds from initial_centroids, then a final assignment.
    Returns (labels [S], centroids [n_clusters, D])."""
    v = _as_f64(v)
    S = v.shape[0]
    k = -(-S // 128) if n_clusters is None else int(n_clusters)
    mu = initial_centroids(v, k)
    for _ in range(rounds):
        mu = update(v, assign(v, mu), mu)
    return assign(v, mu), mu


def stable_permutation(labels) -> np.ndarray:
    """Token order sorted by cluster, ties by token index."""
    return np.argsort(np.asarray(labels), kind="stable")


def objective(v, labels, centroids) -> float:
    """Sum of squared distances of the tokens to their centroids."""
    v = _as_f64(v)
    d = v - np.asarray(centroids, np.float64)[np.asarray(labels)]
    return float((d * d).sum())


def block_energy_removed(v, perm=None, block: int = 128) -> float:
    """Fraction of sum_j |v_j|^2 that subtracting the mean of each block of
    ``block`` consecutive tokens (after ``perm``) takes out."""
    v = _as_f64(v)
    if perm is not None:
        v = v[np.asarray(perm)]
    S = v.shape[0]
    total = float((v * v).sum())
    removed = 0.0
    for b0 in range(0, S, block):
        blk = v[b0:b0 + block]
        m = blk.mean(axis=0)
        removed += blk.shape[0] * float((m * m).sum())
    return removed / total
