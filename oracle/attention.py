"""The plain definition of full spatiotemporal self-attention, in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed
----------------
A video clip is flattened into one sequence of spatiotemporal tokens and full
(non-causal) self-attention runs over all of them [VC-Attention article
(aikraft.ru), §01 "why attention became the bottleneck"]; the score matrix is
the quadratic part of the per-layer self-attention cost [real-time video
generation FLOPS article (sudonull.com), FLOP list].  Flash-style tiling only
avoids materialising the S x S matrix and reaches the same result [same
article, "Optymalizacje", FlashAttention item], so the checker is the
definition itself, per (b, h) and query row i:

    O[i, :] = sum_j softmax_j(scale * <q_i, k_j>) * v_j

computed in fp64 from the bf16 inputs widened exactly.  ``scale`` is the
float32 value handed to the kernel, widened.  Rows are independent, so any
subset of rows can be computed exactly at the real sequence length (row
sampling).

Masked variants (block-causal by frame chunks, after the Wave Forcing note
(airadar.tv), summary paragraph; block-sparse tile masks, after the FLOPS
article's sparse-attention item) restrict the sum over j to the allowed keys.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "widen_bf16",
    "attention_head",
    "attention",
    "probabilities",
    "attention_bruteforce",
    "block_causal_allowed",
    "tile_mask_allowed",
]


def widen_bf16(bits) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64, exactly."""
    b = np.asarray(bits)
    if b.dtype != np.uint16:
        raise TypeError("expected uint16 bf16 bit patterns")
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _as_f64(x) -> np.ndarray:
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return widen_bf16(x)
    return x.astype(np.float64, copy=False)


def attention_head(q, k, v, scale: float, rows=None, allowed=None, block: int = 256) -> np.ndarray:
    """O[rows] for one head.  q: [Sq, D], k, v: [Sk, D] (fp64 or bf16 bits).

    ``allowed(rows) -> bool [len(rows), Sk]`` optionally restricts the keys
    each query row attends to; every row must keep at least one key.

    Steps per block of rows (the definition, stabilised by the row maximum,
    which cancels exactly in the ratio):  s = (Q_blk K^T) * scale;
    m = max_j s;  p = exp(s - m);  O = (p V) / sum_j p.
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    scale = float(np.float64(scale))
    Sq = q.shape[0]
    rows = np.arange(Sq) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty((rows.size, v.shape[1]), dtype=np.float64)
    for r0 in range(0, rows.size, block):
        rr = rows[r0:r0 + block]
        s = (q[rr] @ k.T) * scale
        if allowed is not None:
            keep = allowed(rr)
            if not np.all(keep.any(axis=1)):
                raise ValueError("a query row has no allowed key")
            s = np.where(keep, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        p = np.exp(s - m)
        out[r0:r0 + block] = (p @ v) / p.sum(axis=1, keepdims=True)
    return out


def attention(q, k, v, scale: float, rows=None, allowed=None) -> np.ndarray:
    """O for [B, H, S, D] inputs; ``rows`` selects query rows (same for every
    head).  Returns fp64 [B, H, len(rows), D]."""
    q, k, v = np.asarray(q), np.asarray(k), np.asarray(v)
    B, H, S, D = q.shape
    n = S if rows is None else len(rows)
    out = np.empty((B, H, n, D), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            out[b, h] = attention_head(q[b, h], k[b, h], v[b, h], scale, rows, allowed)
    return out


def probabilities(q, k, scale: float) -> np.ndarray:
    """The full attention matrix P = softmax(scale Q K^T) for one small head
    (used by the invariant checks: every row sums to one)."""
    q, k = _as_f64(q), _as_f64(k)
    s = (q @ k.T) * float(scale)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    return p / p.sum(axis=1, keepdims=True)


def attention_bruteforce(q, k, v, scale: float) -> list:
    """Pure-Python loops with math.exp and math.fsum; for S <= 32, D <= 8.

    A second, independent spelling of the definition that takes no row
    blocks, no vectorisation and no max-subtraction shortcut beyond the
    textbook one."""
    q = [[float(x) for x in row] for row in _as_f64(q)]
    k = [[float(x) for x in row] for row in _as_f64(k)]
    v = [[float(x) for x in row] for row in _as_f64(v)]
    out = []
    for qi in q:
        logits = [float(scale) * math.fsum(a * b for a, b in zip(qi, kj)) for kj in k]
        mx = max(logits)
        w = [math.exp(t - mx) for t in logits]
        z = math.fsum(w)
        out.append([math.fsum(w[j] * v[j][d] for j in range(len(v))) / z
                    for d in range(len(v[0]))])
    return out


def block_causal_allowed(S: int, chunk: int):
    """Mask for block-causal attention by chunks of ``chunk`` tokens (a chunk
    is a group of latent frames): query i sees key j iff chunk(j) <= chunk(i).
    After the Wave Forcing note (airadar.tv), summary: later blocks read the
    context of earlier blocks."""
    def allowed(rows):
        rows = np.asarray(rows)
        return (np.arange(S)[None, :] // chunk) <= (rows[:, None] // chunk)
    return allowed


def tile_mask_allowed(S: int, tile_q: int, tile_k: int, mask):
    """Mask from a boolean [ceil(S/tile_q), ceil(S/tile_k)] tile map: query i
    sees key j iff mask[i // tile_q, j // tile_k].  After the FLOPS article's
    sparse-attention item (skip unimportant token pairs, block-sparse)."""
    mask = np.asarray(mask, dtype=bool)

    def allowed(rows):
        rows = np.asarray(rows)
        return mask[rows // tile_q][:, np.arange(S) // tile_k]
    return allowed
