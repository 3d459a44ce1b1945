"""Pins for the V-Smooth block demean of the fp8 checker (VC-Attention
article, section 02: Demean subtracts the per-channel mean of every 128-token
hardware block and quantises only the residual per channel in E4M3; Restore
adds the mean back through the softmax row sums; the mean costs 16 bits per
channel and block).  CPU only."""

import numpy as np
import pytest

from oracle import attention as oa
from oracle import fp8


def _bf16(x):
    """fp32 -> bf16 bits, nearest even, with torch's CPU cast (a library
    routine, independent of the checker's own rounding)."""
    torch = pytest.importorskip("torch")
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_bf16_rne_matches_torch_cast():
    torch = pytest.importorskip("torch")
    g = np.random.default_rng(3)
    x = np.concatenate([
        g.standard_normal(100000).astype(np.float32) * np.float32(2.0) ** g.integers(-30, 30, 100000),
        # exact ties at both parities of the kept bit, and their neighbours
        (np.arange(1, 4097, dtype=np.uint32) << 16 | np.uint32(0x8000)).view(np.float32),
        (np.arange(1, 4097, dtype=np.uint32) << 16 | np.uint32(0x7FFF)).view(np.float32),
        (np.arange(1, 4097, dtype=np.uint32) << 16 | np.uint32(0x8001)).view(np.float32),
    ]).astype(np.float32)
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(fp8.bf16_rne(x), ref)


def test_block_means_closed_form_with_ties():
    """V = token index in every channel for the first 256 tokens and
    2 (t - 256) for a ragged third block of 44 tokens (all exact in bf16):
    block means 63.5, 191.5 and 43; rounded to bf16 they are 63.5, 192 (a tie
    at spacing 1, to the even mantissa) and 43.  Residuals are taken against
    the rounded means."""
    S, D = 300, 128
    t = np.arange(S, dtype=np.float32)
    t[256:] = 2 * (t[256:] - 256)
    t = t[:, None] * np.ones((1, D), np.float32)
    z = fp8.quantize_head(_bf16(t), _bf16(t), _bf16(t), v_mean="block")
    assert "v_mean" not in z
    np.testing.assert_array_equal(z["v_bmean"], np.repeat([[63.5], [192.0], [43.0]], D, axis=1))
    res = t - np.repeat(z["v_bmean"], 128, axis=0)[:S]
    amax = np.abs(res).max(axis=0)
    assert np.all(amax == 64.0)  # block 1: |128 - 192| = 64
    np.testing.assert_array_equal(z["v_scale"], np.full(D, np.float32(64.0 / 448.0)))
    np.testing.assert_array_equal(z["v8"], fp8.e4m3_encode(np.clip(
        (res * np.float32(448.0 / 64.0)).astype(np.float32), -448, 448)))


def test_constant_blocks_quantise_to_zero_and_restore_exactly():
    """A V that is constant within every 128-token block leaves no residual:
    zero codes, unit scales, the block constants as means, and (without P
    quantisation) the model equals the definition on V itself."""
    g = np.random.default_rng(1)
    S, D = 333, 128
    nbv = -(-S // 128)
    c = np.round(g.standard_normal((nbv, D)) * 8) / 4  # exact in bf16
    v = np.repeat(c, 128, axis=0)[:S].astype(np.float32)
    q = g.standard_normal((S, D)).astype(np.float32)
    k = g.standard_normal((S, D)).astype(np.float32)
    z = fp8.quantize_head(_bf16(q), _bf16(k), _bf16(v), v_mean="block")
    # codes decode to zero (a -0.0 input minus a +0.0 mean gives code -0)
    assert np.all(fp8.e4m3_decode(z["v8"]) == 0) and np.all(z["v_scale"] == 1.0)
    np.testing.assert_array_equal(z["v_bmean"], c.astype(np.float32))
    got = fp8.attention_fp8_model_head(z, 0.09, p_quant=False)
    blk = np.arange(S) // 64
    qh = fp8.e4m3_decode(z["q8"]) * z["q_scale"][blk][:, None].astype(np.float64)
    kh = fp8.e4m3_decode(z["k8"]) * z["k_scale"][blk][:, None].astype(np.float64) + z["k_mean"][blk]
    ref = oa.attention_head(qh, kh, v.astype(np.float64), 0.09)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_per_block_offsets_change_only_the_means():
    """Adding a constant per (block, channel) to V shifts that block's mean by
    the constant and leaves codes and scales unchanged: Demean removes block
    offsets before quantisation.  Values are multiples of 1/16 below 16 in
    magnitude, so V, V + offset and every mean are exact in bf16; each block
    is made of +-x pairs so its mean is the offset exactly."""
    g = np.random.default_rng(2)
    S, D = 512, 128
    nbv = S // 128
    x = np.round(g.uniform(-3.5, 3.5, (nbv, 64, D)) * 16) / 16
    blocks = np.concatenate([x, -x], axis=1)
    for b in range(nbv):
        blocks[b] = blocks[b][g.permutation(128)]
    v0 = blocks.reshape(S, D).astype(np.float32)
    off = (g.integers(-8, 9, (nbv, D))).astype(np.float32)
    v1 = v0 + np.repeat(off, 128, axis=0)
    q = _bf16(g.standard_normal((S, D)).astype(np.float32))
    z0 = fp8.quantize_head(q, q, _bf16(v0), v_mean="block")
    z1 = fp8.quantize_head(q, q, _bf16(v1), v_mean="block")
    np.testing.assert_array_equal(z0["v_bmean"], np.zeros((nbv, D), np.float32))
    np.testing.assert_array_equal(z1["v_bmean"], off)
    # equal codes up to the sign of zero residuals (-0.0 + offset is +0.0)
    np.testing.assert_array_equal(fp8.e4m3_decode(z0["v8"]), fp8.e4m3_decode(z1["v8"]))
    np.testing.assert_array_equal(z0["v_scale"], z1["v_scale"])
    # the global mean cannot remove them: its residual spread grows
    zg = fp8.quantize_head(q, q, _bf16(v1), v_mean="global")
    assert np.all(zg["v_scale"] >= z1["v_scale"])
    assert np.mean(zg["v_scale"] > z1["v_scale"]) > 0.9


def test_model_without_p_quantisation_is_sdpa_on_restored_values():
    """Library routine special case: with P unquantised the block-demean model
    is textbook attention (torch fp64 SDPA) on Q_hat, K_hat + k_mean and
    V_hat + v_bmean of each key's 128-token block."""
    torch = pytest.importorskip("torch")
    g = np.random.default_rng(4)
    S, D = 300, 128
    nb, nbv = -(-S // 64), -(-S // 128)
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])
    z = {
        "q8": g.choice(finite, (S, D)).astype(np.uint8),
        "k8": g.choice(finite, (S, D)).astype(np.uint8),
        "v8": g.choice(finite, (S, D)).astype(np.uint8),
        "q_scale": (g.uniform(0.5, 2, nb) / 448).astype(np.float32),
        "k_scale": (g.uniform(0.5, 2, nb) / 448).astype(np.float32),
        "k_mean": g.standard_normal((nb, D)).astype(np.float32),
        "v_bmean": g.standard_normal((nbv, D)).astype(np.float32),
        "v_scale": (g.uniform(0.5, 2, D) / 448).astype(np.float32),
    }
    blk = np.arange(S) // 64
    qh = fp8.e4m3_decode(z["q8"]) * z["q_scale"][blk][:, None].astype(np.float64)
    kh = fp8.e4m3_decode(z["k8"]) * z["k_scale"][blk][:, None].astype(np.float64) + z["k_mean"][blk]
    vh = (fp8.e4m3_decode(z["v8"]) * z["v_scale"][None, :].astype(np.float64)
          + z["v_bmean"][np.arange(S) // 128].astype(np.float64))
    scale = float(np.float32(0.088388))
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(np.ascontiguousarray(t))[None, None] for t in (qh, kh, vh)), scale=scale)[0, 0].numpy()
    got = fp8.attention_fp8_model_head(z, scale, p_quant=False)
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-11)


def test_quantised_weights_bruteforce_tiny():
    """Pure-Python loops over a tiny head (S = 200, D = 128, two 128-blocks):
    weights from the exact E4M3 cast of 448 * 2^(t - M), row sum of the
    weights, each block's weight sum times its mean."""
    import math
    g = np.random.default_rng(5)
    S, D = 200, 128
    q = _bf16(g.standard_normal((S, D)).astype(np.float32))
    k = _bf16(g.standard_normal((S, D)).astype(np.float32))
    v = _bf16((g.standard_normal((S, D)) + 3 * (np.arange(S)[:, None] >= 128)).astype(np.float32))
    z = fp8.quantize_head(q, k, v, v_mean="block")
    rows = [0, 77, 199]
    got = fp8.attention_fp8_model_head(z, 0.1, rows=rows)
    dq = fp8.e4m3_decode
    for n, i in enumerate(rows):
        bi = i // 64
        qi = [float(dq(z["q8"][i, d])) * float(z["q_scale"][bi]) for d in range(D)]
        ts = []
        for j in range(S):
            bj = j // 64
            kj = [float(dq(z["k8"][j, d])) * float(z["k_scale"][bj]) + float(z["k_mean"][bj, d])
                  for d in range(D)]
            ts.append(0.1 * math.fsum(a * b for a, b in zip(qi, kj)) / math.log(2.0))
        M = math.ceil(max(ts))
        w = [float(dq(fp8.e4m3_encode(np.array([448.0 * 2.0 ** (t - M)]))[0])) / 448.0 for t in ts]
        l = math.fsum(w)
        for d in (0, 5, 127):
            acc = math.fsum(w[j] * float(dq(z["v8"][j, d])) for j in range(S)) * float(z["v_scale"][d])
            mean_part = math.fsum(math.fsum(w[j] for j in range(b * 128, min(S, b * 128 + 128)))
                                  * float(z["v_bmean"][b, d]) for b in range(2))
            o = (acc + mean_part) / l
            assert abs(got[n, d] - o) <= 1e-12 * (1 + abs(o)), (i, d, got[n, d], o)
