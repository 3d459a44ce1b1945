"""fp8 (E4M3) low-bit attention: format, pre-pass and quantisation model.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources on the pages
--------------------
* FP8 doubles tensor throughput [real-time video generation FLOPS article
  (sudonull.com), "Optymalizacje", FP8 item].
* Q/K smoothing before the low-bit QK^T (the SageAttention2 approach) and
  the value term as the remaining error [VC-Attention article (aikraft.ru),
  §01].
* V-Smooth: subtract a mean, quantise only the residual per channel in
  E4M3, add the mean back using the online-softmax row sum, no second pass
  [VC-Attention article, §02, Demean and Restore].  The article's own mean
  is taken over each hardware block of 128 tokens and costs 0.125 bit per
  value element, i.e. 16 bits per channel per block [same section].
* The E4M3 byte read as an integer is close to 8*log2(v) + 56; ExpCast-FP8
  writes the byte of a softmax weight from its log-domain score with one
  multiply-add and the centring constant -0.35; it matches the exp-then-cast
  byte in 79.6% of cases per doubling and is otherwise one code off; the
  per-row total variation stays under 3.64% plus underflow tails
  [VC-Attention article, §03].

Readings taken where the pages are silent: Q and K use one scale per
64-token block; K is smoothed by the mean of each 64-token block (or one
global mean per head), and the per-block mean is compensated exactly by
adding q_hat . k_mean_b to the scores of block b; V is smoothed by one per-
channel mean over the sequence with one per-channel scale, or (the article's
Demean, ``v_mean="block"``) by the per-channel mean of each 128-token block
(valid tokens only) rounded to bf16 (the 16-bit mean), with one per-channel
scale of the residual over the sequence; P is quantised as E4M3(448 * 2^(t -
M)) where t is the log2-domain score and M the integer ceiling of the row
maximum of t; the row sum is the sum of the quantised weights (so the
weights of a row sum to one and the mean restore is exact); ExpCast takes the
byte position z = 8 (t - M) + 8 log2(448) + 55.65 and rounds the value the
byte map gives to z (exponent floor(z/8) - 7, mantissa 1 + (z mod 8)/8) to
E4M3: in the normal range that is round-half-even(z) itself, below it the
nearest subnormal code (the pages leave the underflow open).

Precision of the integer-valued decisions (codes): the pre-pass takes them
in the precision the kernel takes them in, so the codes can be compared bit
for bit:  means are fp64 sums of the bf16 inputs (exact here) divided in
fp64 and rounded once to fp32;  residual = fp32(x - mean);  amax = max|r|;
scale = fp32(amax / 448) and inv = fp32(448 / amax) (both from fp64
quotients), or 1 and 0 when amax = 0;  code = E4M3_RNE(clamp(fp32(r * inv),
-448, 448)).  The 16-bit block mean of V is bf16_rne(fp32 mean) and the
residual is taken against that rounded mean, fp32(x - mean16), so that
adding it back restores exactly what was subtracted.
"""

from __future__ import annotations

import math

import numpy as np

from .attention import _as_f64

__all__ = [
    "E4M3_MAX",
    "e4m3_encode",
    "e4m3_decode",
    "e4m3_table",
    "quantize_head",
    "quantize",
    "attention_fp8_model_head",
    "attention_fp8_model",
    "cosine",
    "max_abs",
    "mean_rel_l1",
]

E4M3_MAX = 448.0
_MIN_NORMAL = 2.0 ** -6


def e4m3_table() -> np.ndarray:
    """Value of each of the 256 E4M3 codes, from the format definition:
    1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field
    0 holds subnormals m * 2^-9; 0x7F / 0xFF are NaN; there is no infinity."""
    vals = np.empty(256, dtype=np.float64)
    for c in range(256):
        sign = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            vals[c] = np.nan
        elif e == 0:
            vals[c] = sign * m * 2.0 ** -9
        else:
            vals[c] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_TABLE = e4m3_table()


def e4m3_decode(codes) -> np.ndarray:
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(x) -> np.ndarray:
    """Round to the nearest E4M3 value, ties to even mantissa, after clamping
    to +-448 (saturation).  Input is any float array (taken exactly in fp64);
    output uint8 codes.  Negative values that round to zero give 0x80."""
    x = np.asarray(x, dtype=np.float64)
    neg = np.signbit(x)
    a = np.minimum(np.abs(x), E4M3_MAX)
    code = np.zeros(a.shape, dtype=np.int64)
    sub = a < _MIN_NORMAL
    # subnormal range: multiples of 2^-9 (a * 2^9 is exact, rint is RNE)
    code[sub] = np.rint(a[sub] * 2.0 ** 9).astype(np.int64)  # 8 -> 0x08, the least normal
    nrm = ~sub
    f, E = np.frexp(a[nrm])            # a = f * 2^E, f in [0.5, 1)
    e = E.astype(np.int64) - 1         # a = s * 2^e, s in [1, 2)
    s = f * 2.0                        # exact
    mant = np.rint((s - 1.0) * 8.0).astype(np.int64)  # exact scaling, RNE
    carry = mant == 8
    e = e + carry
    mant = np.where(carry, 0, mant)
    code[nrm] = ((e + 7) << 3) | mant
    code = np.where(np.isnan(x), 0x7F, code)
    return (code | (neg.astype(np.int64) << 7)).astype(np.uint8)


def _scales(amax: np.ndarray):
    """scale = fp32(amax/448), inv = fp32(448/amax); (1, 0) where amax == 0."""
    amax = np.asarray(amax, dtype=np.float32).astype(np.float64)
    zero = amax == 0.0
    safe = np.where(zero, 1.0, amax)
    scale = np.where(zero, 1.0, safe / E4M3_MAX).astype(np.float32)
    inv = np.where(zero, 0.0, E4M3_MAX / safe).astype(np.float32)
    return scale, inv


def _codes(r32: np.ndarray, inv32) -> np.ndarray:
    """E4M3 codes of fp32(r * inv) clamped to +-448 (fp32 product, RNE)."""
    prod = (r32.astype(np.float32) * np.asarray(inv32, dtype=np.float32)).astype(np.float32)
    return e4m3_encode(np.clip(prod, -E4M3_MAX, E4M3_MAX))


def bf16_rne(x32) -> np.ndarray:
    """Round float32 values to bfloat16, nearest even, returned as float32
    (finite inputs): keep the top 16 bits of the fp32 pattern after adding
    0x7FFF plus the lowest kept bit."""
    u = np.asarray(x32, np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def _mean32(x32: np.ndarray, axis: int) -> np.ndarray:
    """fp32(fp64 sum / n): the sum of bf16 values is exact in fp64 here."""
    n = x32.shape[axis]
    s = x32.astype(np.float64).sum(axis=axis)
    return (s / float(n)).astype(np.float32)


def quantize_head(q, k, v, block: int = 64, k_mean: str = "block", v_mean: str = "global",
                  v_block: int = 128):
    """fp8 pre-pass for one (b, h).  q, k, v: bf16 bits or exact values [S, D].

    Returns a dict with uint8 codes q8, k8, v8 [S, D]; q_scale, k_scale
    [nb] (nb = ceil(S / block)); k_mean [nb or 1, D]; v_mean, v_scale [D]
    (all float32).  ``k_mean`` is "block" (one mean per block of ``block``
    tokens, statistics over the valid tokens only) or "global" (one mean
    per channel over the whole sequence).  ``v_mean`` is "global" (v_mean
    [D]) or "block" (V-Smooth Demean: v_bmean [ceil(S / v_block), D], the
    bf16-rounded per-channel mean of each block of ``v_block`` tokens, as
    float32; v_mean is then absent)."""
    q32 = _as_f64(q).astype(np.float32)
    k32 = _as_f64(k).astype(np.float32)
    v32 = _as_f64(v).astype(np.float32)
    S, D = q32.shape
    nb = -(-S // block)
    out = {
        "q8": np.empty((S, D), np.uint8), "k8": np.empty((S, D), np.uint8),
        "q_scale": np.empty(nb, np.float32), "k_scale": np.empty(nb, np.float32),
    }
    if k_mean == "block":
        kmean = np.empty((nb, D), np.float32)
        for b in range(nb):
            kmean[b] = _mean32(k32[b * block:(b + 1) * block], axis=0)
        kmean_tok = np.repeat(kmean, block, axis=0)[:S]
    elif k_mean == "global":
        kmean = _mean32(k32, axis=0)[None, :]
        kmean_tok = np.broadcast_to(kmean, (S, D))
    else:
        raise ValueError(k_mean)
    kres = (k32 - kmean_tok).astype(np.float32)
    for b in range(nb):
        sl = slice(b * block, min(S, (b + 1) * block))
        for name, src, dst in (("q", q32, "q8"), ("k", kres, "k8")):
            amax = np.max(np.abs(src[sl]))
            sc, inv = _scales(amax)
            out[name + "_scale"][b] = sc
            out[dst][sl] = _codes(src[sl], inv)
    out["k_mean"] = kmean
    if v_mean == "global":
        vmean = _mean32(v32, axis=0)
        vres = (v32 - vmean[None, :]).astype(np.float32)
        out["v_mean"] = vmean
    elif v_mean == "block":
        nbv = -(-S // v_block)
        vbm = np.empty((nbv, D), np.float32)
        for b in range(nbv):
            vbm[b] = bf16_rne(_mean32(v32[b * v_block:(b + 1) * v_block], axis=0))
        vres = (v32 - np.repeat(vbm, v_block, axis=0)[:S]).astype(np.float32)
        out["v_bmean"] = vbm
    else:
        raise ValueError(v_mean)
    vsc, vinv = _scales(np.max(np.abs(vres), axis=0))
    out["v_scale"] = vsc
    out["v8"] = _codes(vres, vinv[None, :])
    return out


def quantize(q, k, v, block: int = 64, k_mean: str = "block", v_mean: str = "global"):
    """quantize_head over [B, H, S, D]; arrays gain leading [B, H] axes."""
    q, k, v = np.asarray(q), np.asarray(k), np.asarray(v)
    B, H = q.shape[:2]
    parts = [[quantize_head(q[b, h], k[b, h], v[b, h], block, k_mean, v_mean) for h in range(H)]
             for b in range(B)]
    return {key: np.stack([np.stack([parts[b][h][key] for h in range(H)]) for b in range(B)])
            for key in parts[0][0]}


# ExpCast-FP8 (VC-Attention article, section 03): the E4M3 byte of a value
# v, read as an integer, is about 8 log2(v) + 56; the article writes the byte
# of a weight directly from its log-domain score with one multiply-add and a
# centring constant beta = -0.35.  Here the weight is 448 p with log2 p =
# t - M, so its byte position is z = 8 (t - M) + 8 log2(448) + 56 - 0.35
# (t <= M keeps z <= 126.1, below 126.5: at most the code of 448).
EXPCAST_BETA = -0.35
EXPCAST_OFFSET = 8.0 * math.log2(E4M3_MAX) + 56.0 + EXPCAST_BETA


def byte_map_value(z) -> np.ndarray:
    """The value the E4M3 byte map gives to a real byte position z.

    A normal E4M3 byte read as an integer is 8 e + m for the value
    2^(e - 7) (1 + m / 8) (exponent field e, mantissa field m), which is why
    the byte is close to 8 log2(v) + 56 (VC-Attention article, section 03).
    The same rule for every real z: 2^(floor(z / 8) - 7) (1 + (z mod 8) / 8);
    -inf gives 0.  It is exact at the bytes 8 .. 126 and commutes with powers
    of two: byte_map_value(z + 8 k) = 2^k byte_map_value(z)."""
    z = np.asarray(z, np.float64)
    with np.errstate(invalid="ignore"):
        e = np.floor(z / 8.0)
        f = z / 8.0 - e
        e = np.where(np.isfinite(e), e, 0.0)
        val = np.ldexp(1.0 + f, (e - 7.0).astype(np.int64))
    return np.where(np.isneginf(z), 0.0, val)


def expcast_byte(log2_v) -> np.ndarray:
    """ExpCast code of a value given by its base-2 logarithm (no P scale).

    The byte position is z = 8 log2(v) + 56 - 0.35 (one multiply-add); the
    code is the E4M3 rounding (nearest, ties to even, saturating at 448) of
    byte_map_value(z).  Wherever z >= 7.5 that is round-half-even(z), the
    article's conversion to an integer.  Below that the position has no E4M3
    code of its own (codes 1 .. 7 are the subnormals m 2^-9, not on the log
    map), and the code is the subnormal nearest the byte map's value: one
    code or less from the exact cast, as in the normal range."""
    z = 8.0 * np.asarray(log2_v, np.float64) + 56.0 + EXPCAST_BETA
    return e4m3_encode(byte_map_value(z))


def attention_fp8_model_head(qz: dict, scale: float, rows=None, block: int = 64,
                             p_quant: bool = True, p_scale: float = E4M3_MAX,
                             chunk: int = 256, p_cast: str = "exp",
                             v_block: int = 128, allowed=None) -> np.ndarray:
    """Quantisation model of the fp8 attention for one head, in fp64.

    Steps: dequantise Q_hat = dec(q8) q_scale, K_hat = dec(k8) k_scale,
    V_hat = dec(v8) v_scale;  s_ij = scale (Q_hat_i . K_hat_j + Q_hat_i .
    k_mean_b(j));  t = log2(e) s;  M_i = ceil(max_j t_ij);  p = 2^(t - M);
    w = dec(E4M3(p_scale p)) / p_scale (or w = p without P quantisation;
    with p_cast="expcast" the E4M3 byte is the ExpCast byte of p_scale p,
    expcast_byte(t - M + log2(p_scale)));
    l_i = sum_j w_ij;  O_i = (sum_j w_ij V_hat_j) / l_i + v_mean.
    ``allowed(rows) -> bool [len(rows), S]`` restricts each row to its allowed
    keys (block-causal or block-sparse masks): the others score -inf and
    weigh 0, and M is the maximum over the allowed keys.
    With block means (``v_bmean`` in qz, V-Smooth Demean) the mean is
    restored per key instead: O_i = sum_j w_ij (V_hat_j + v_bmean_b(j)) / l_i,
    b(j) = j // v_block (the row sum of each block's weights times its mean).

    The weights are taken against the row maximum M, as the definition
    of the softmax has it.  An online kernel takes them against a running
    reference that rises by whole powers of two and rescales its sums; for
    both casts (exp-then-cast and ExpCast, whose byte map commutes with
    powers of two) that gives the same weights except where E4M3 rounds to
    a subnormal, i.e. for weights below 2^-6 / 448 (about 2^-14.8).
    The row sum is that of the weights actually applied to V, so each row's
    weights sum to one and the mean restore of the VC-Attention article
    (section 02, Restore: sum_j P_j v_mean / l = v_mean) holds exactly.
    """
    S, D = qz["q8"].shape
    nb = qz["q_scale"].shape[0]
    tok_blk = np.arange(S) // block
    qh = e4m3_decode(qz["q8"]) * qz["q_scale"].astype(np.float64)[tok_blk][:, None]
    kh = e4m3_decode(qz["k8"]) * qz["k_scale"].astype(np.float64)[tok_blk][:, None]
    vh = e4m3_decode(qz["v8"]) * qz["v_scale"].astype(np.float64)[None, :]
    if "v_bmean" in qz:
        vbm = qz["v_bmean"].astype(np.float64)
        vh = vh + np.repeat(vbm, v_block, axis=0)[:S]
        vm_add = np.zeros((1, D))
    else:
        vm_add = qz["v_mean"].astype(np.float64)[None, :]
    km = qz["k_mean"].astype(np.float64)
    kmean_tok = km[tok_blk] if km.shape[0] == nb and nb > 1 else np.broadcast_to(km[0], (S, D))
    keff = kh + kmean_tok          # q.(k_res + k_mean) = q.k_res + q.k_mean
    rows = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty((rows.size, D), np.float64)
    log2e = 1.0 / math.log(2.0)

    def weights(t, M):
        # masked scores (-inf) weigh 0, also before any allowed key is seen
        d = np.where(np.isneginf(t), -np.inf, t - M)
        if p_cast == "expcast":
            return e4m3_decode(expcast_byte(d + math.log2(p_scale))) / p_scale
        p = np.exp2(d)
        return e4m3_decode(e4m3_encode(p * p_scale)) / p_scale if p_quant else p

    # -inf - -inf (a masked key before any allowed one) is discarded by np.where
    with np.errstate(invalid="ignore"):
        for r0 in range(0, rows.size, chunk):
            rr = rows[r0:r0 + chunk]
            t = (qh[rr] @ keff.T) * (float(np.float64(scale)) * log2e)
            if allowed is not None:
                t = np.where(allowed(rr), t, -np.inf)
            M = np.ceil(t.max(axis=1, keepdims=True))
            w = weights(t, M)
            l = w.sum(axis=1, keepdims=True)
            out[r0:r0 + chunk] = (w @ vh) / l + vm_add
    return out


def attention_fp8_model(qz: dict, scale: float, rows=None, **kw) -> np.ndarray:
    """attention_fp8_model_head over the [B, H] axes of ``quantize`` output."""
    B, H = qz["q8"].shape[:2]
    n = qz["q8"].shape[2] if rows is None else len(rows)
    out = np.empty((B, H, n, qz["q8"].shape[3]), np.float64)
    for b in range(B):
        for h in range(H):
            out[b, h] = attention_fp8_model_head({key: val[b, h] for key, val in qz.items()},
                                                 scale, rows, **kw)
    return out


# Error measures used by the tolerance checks (fp64 sums).
def cosine(a, b) -> float:
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    return float(a @ b / math.sqrt(float(a @ a) * float(b @ b)))


def max_abs(a, b) -> float:
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))


def mean_rel_l1(a, ref) -> float:
    """sum |a - ref| / sum |ref| (robust near zero)."""
    a = np.asarray(a, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.abs(a - ref).sum() / np.abs(ref).sum())
