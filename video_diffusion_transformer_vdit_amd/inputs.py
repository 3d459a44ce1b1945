"""Seeded synthetic inputs for spatiotemporal self-attention.

This module only draws random numbers and rounds them to bfloat16; it holds
none of the attention arithmetic, so both the HIP path and the fp64 checker
can consume its output.

Workload shapes follow the token-count rule of the pages: a clip is flattened
into latent frames x tokens per frame (FLOP-accounting page, intro: 21 latent
frames x 3,600 tokens = 75,600 tokens for 5 s of 720p video), with H heads of
width D = 128 (model width 5120 = 40 x 128).  No real activations exist here,
so every tensor is Gaussian with the structure each workload names.

Recipe (identical on every machine, independent of thread count):

* Each (tensor, batch b, head h) plane of shape [S, D] is drawn from its own
  PCG64 stream seeded with ``SeedSequence([seed, t, b, h])`` where t = 0, 1, 2
  for Q, K, V: ``standard_normal((S, D), float32)``.
* Structure draws use their own streams:
  - ``k_offset``: per-(head, channel) offset c[h, d] ~ N(0, 0.5) (0.5 is the
    standard deviation) from ``SeedSequence([seed, 3, h])``, added to every
    K token of that head, shared across the batch.
  - ``outlier``: per head, 4 distinct channels chosen from
    ``SeedSequence([seed, 4, h])``; those channels of K and V (the same
    indices for both) are multiplied by 8.
* The float32 result is rounded to bfloat16 with round-to-nearest-even.  The
  bf16 values are the ground truth for every consumer.
"""

from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "get_workload",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "make_plane",
    "make_head",
    "make_inputs",
    "outlier_channels",
    "k_offsets",
    "make_block_mask",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    S: int
    D: int
    structure: str  # "iid" | "k_offset" | "outlier"
    seed: int
    frames: int
    tokens_per_frame: int
    note: str

    @property
    def flop(self) -> int:
        """Attention-core FLOPs: QK^T and PV, 2 flop per multiply-add each."""
        return 4 * self.B * self.H * self.S * self.S * self.D

    @property
    def shape(self):
        return (self.B, self.H, self.S, self.D)


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny-3x16x16", 1, 2, 768, 128, "iid", 1, 3, 256,
                 "3 latent frames of 16x16 tokens; small enough for the fp64 checker in full"),
        Workload("wan2.1-1.3b-480p", 1, 12, 32760, 128, "k_offset", 2, 21, 1560,
                 "832x480, 81 frames: 21 latent frames x 30x52 patches; K carries a per-channel offset"),
        Workload("wan2.2-720p-16x", 1, 40, 18900, 128, "iid", 3, 21, 900,
                 "720p with a 16x16-compressing VAE: 21 x 900 tokens (nominal)"),
        Workload("wan2.1-14b-720p", 1, 40, 75600, 128, "outlier", 4, 21, 3600,
                 "1280x720, 81 frames: 21 latent frames x 80x45 tokens; 4 outlier channels per head x8 in K and V"),
    ]
}
# The low-bit workload quantises exactly the tensors of the 720p 14B workload.
WORKLOADS["wan2.1-14b-720p-fp8"] = dataclasses.replace(
    WORKLOADS["wan2.1-14b-720p"], name="wan2.1-14b-720p-fp8",
    note="same seeded tensors as wan2.1-14b-720p, fed through the fp8 pre-pass")


def get_workload(name: str) -> Workload:
    try:
        return WORKLOADS[name]
    except KeyError:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(WORKLOADS)}") from None


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits.

    Inputs here are finite Gaussians, so NaN/Inf handling is not needed.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bits to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def outlier_channels(w: Workload, h: int, n: int = 4) -> np.ndarray:
    rng = np.random.default_rng([w.seed, 4, h])
    return np.sort(rng.choice(w.D, size=n, replace=False))


def k_offsets(w: Workload, h: int) -> np.ndarray:
    rng = np.random.default_rng([w.seed, 3, h])
    return rng.normal(0.0, 0.5, size=w.D).astype(np.float32)


def make_plane(w: Workload, tensor: str, b: int, h: int, S: int | None = None) -> np.ndarray:
    """bf16 bits [S, D] of one (tensor, b, h) plane.

    A shorter ``S`` returns the first S rows of the full-length plane (the
    normal stream is consumed row by row), which the shape sweeps use."""
    t = {"q": 0, "k": 1, "v": 2}[tensor]
    S = w.S if S is None else S
    rng = np.random.default_rng([w.seed, t, b, h])
    x = rng.standard_normal((S, w.D), dtype=np.float32)
    if w.structure == "k_offset" and tensor == "k":
        x += k_offsets(w, h)[None, :]
    elif w.structure == "outlier" and tensor in ("k", "v"):
        x[:, outlier_channels(w, h)] *= np.float32(8.0)
    elif w.structure not in ("iid", "k_offset", "outlier"):
        raise ValueError(f"unknown structure {w.structure!r}")
    return f32_to_bf16_bits(x)


def make_head(w: Workload, b: int, h: int):
    """(q, k, v) bf16 bits, each [S, D], for one (b, h)."""
    return tuple(make_plane(w, t, b, h) for t in ("q", "k", "v"))


def make_inputs(w: Workload | str, threads: int = 8):
    """Full (q, k, v) bf16 bits, each [B, H, S, D] uint16, C-contiguous."""
    if isinstance(w, str):
        w = get_workload(w)
    out = {t: np.empty(w.shape, dtype=np.uint16) for t in ("q", "k", "v")}

    def job(args):
        t, b, h = args
        out[t][b, h] = make_plane(w, t, b, h)

    jobs = [(t, b, h) for t in ("q", "k", "v") for b in range(w.B) for h in range(w.H)]
    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        list(ex.map(job, jobs))
    return out["q"], out["k"], out["v"]


def make_block_mask(B: int, H: int, S: int, density: float, seed: int,
                    q_group: int = 256, q_block: int = 128, k_tile: int = 64) -> np.ndarray:
    """Seeded block-sparse map, uint8 [B, H, ceil(S/q_block), ceil(S/k_tile)].

    Stand-in for a learned or score-based selection (sparse attention that
    skips unimportant token pairs): for every group of ``q_group`` queries a
    ``density`` fraction of the key tiles is drawn uniformly at random, plus
    the tiles holding the group's own tokens, and every ``q_block`` row block
    of the group takes that selection.  Every row block keeps at least one
    key tile."""
    g = np.random.default_rng(seed)
    nqb = -(-S // q_block)
    nkt = -(-S // k_tile)
    per = q_group // q_block
    ngroups = -(-nqb // per)
    mask = np.zeros((B, H, nqb, nkt), np.uint8)
    n_pick = max(1, int(round(density * nkt)))
    for b in range(B):
        for h in range(H):
            for gi in range(ngroups):
                sel = np.zeros(nkt, bool)
                sel[g.choice(nkt, n_pick, replace=False)] = True
                lo = gi * q_group // k_tile
                hi = min(nkt, -(-min(S, (gi + 1) * q_group) // k_tile))
                sel[lo:hi] = True
                mask[b, h, gi * per:(gi + 1) * per] = sel
    return mask
