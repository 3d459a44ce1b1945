"""Pins for the fp8 part of the checker: the E4M3 encoder against the format
definition, the page's byte/log2 relation and torch's CPU cast; the pre-pass
against closed forms and error bounds; the quantisation model against torch's
fp64 SDPA on dequantised operands.  CPU only."""

import math
import os

import numpy as np
import pytest

from oracle import attention as oa
from oracle import fp8

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
FINITE = [c for c in range(256) if (c & 0x7F) != 0x7F]


def test_golden_codes():
    n = 0
    with open(os.path.join(GOLDEN, "e4m3_codes.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            val, code, _src = line.split()
            assert int(fp8.e4m3_encode(np.array([float(val)]))[0]) == int(code, 16), line
            assert fp8.e4m3_decode(np.array([int(code, 16)]))[0] == float(val), line
            n += 1
    assert n >= 10


def test_roundtrip_every_finite_code():
    vals = fp8.e4m3_decode(np.array(FINITE))
    codes = fp8.e4m3_encode(vals)
    assert codes.tolist() == FINITE


def test_table_is_monotone_and_spans_the_format():
    pos = fp8.e4m3_decode(np.arange(0, 0x7F))
    assert np.all(np.diff(pos) > 0)
    assert pos[-1] == 448.0 and pos[1] == 2.0 ** -9 and pos[8] == 2.0 ** -6
    assert np.isnan(fp8.e4m3_decode(np.array([0x7F, 0xFF]))).all()


def test_ties_go_to_even_mantissa():
    for c in range(0, 0x7E):
        lo, hi = fp8.e4m3_decode(np.array([c, c + 1]))
        mid = (lo + hi) / 2
        even = c if c % 2 == 0 else c + 1
        assert fp8.e4m3_encode(np.array([mid]))[0] == even, c
        assert fp8.e4m3_encode(np.array([np.nextafter(mid, 0)]))[0] == c
        assert fp8.e4m3_encode(np.array([np.nextafter(mid, 1e9)]))[0] == c + 1
        assert fp8.e4m3_encode(np.array([-mid]))[0] == (even | 0x80)


def test_saturation_and_zero():
    assert fp8.e4m3_encode(np.array([449.0, 1e6, 464.0, -1e9])).tolist() == [0x7E, 0x7E, 0x7E, 0xFE]
    assert fp8.e4m3_encode(np.array([0.0, 2.0 ** -11, -2.0 ** -11])).tolist() == [0x00, 0x00, 0x80]


def test_matches_torch_cpu_cast_in_range():
    """Library routine special case: torch's float8_e4m3fn CPU cast (RNE) on
    values inside +-448, including every midpoint between codes."""
    torch = pytest.importorskip("torch")
    g = np.random.default_rng(0)
    x = np.concatenate([
        g.standard_normal(200000) * 30,
        g.standard_normal(50000) * 0.01,
        np.exp2(g.uniform(-12, 8.8, 50000)) * np.sign(g.standard_normal(50000)),
    ]).astype(np.float32)
    v = fp8.e4m3_decode(np.array(FINITE[:0x7E]))
    x = np.concatenate([x, ((v[:-1] + v[1:]) / 2).astype(np.float32)])
    x = np.clip(x, -448, 448)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = fp8.e4m3_encode(x)
    assert np.array_equal(got, ref)


def test_byte_is_about_8_log2_plus_56():
    """VC-Attention article, section 03: the byte read as an integer is close
    to 8*log2(v) + 56 (exact at powers of two, within about one code elsewhere)."""
    v = np.exp2(np.linspace(-6, math.log2(448), 5000))
    codes = fp8.e4m3_encode(v).astype(np.float64)
    d = codes - (8 * np.log2(v) + 56)
    assert np.all(np.abs(d) <= 1.2)
    p2 = np.exp2(np.arange(-6, 9)).astype(np.float64)
    assert np.array_equal(fp8.e4m3_encode(p2).astype(np.float64), 8 * np.log2(p2) + 56)


def _bf16(x):
    from video_diffusion_transformer_vdit_amd.inputs import f32_to_bf16_bits
    return f32_to_bf16_bits(np.asarray(x, np.float32))


def test_constant_block_gives_unit_scale_zero_codes():
    S, D = 150, 128
    q = _bf16(np.full((S, D), 0.75))
    k = _bf16(np.full((S, D), -2.5))
    v = _bf16(np.tile(np.linspace(-3, 3, D), (S, 1)))
    z = fp8.quantize_head(q, k, v)
    assert np.all(z["k8"] == 0) and np.all(z["k_scale"] == 1.0)
    assert np.all(z["k_mean"] == np.float32(-2.5))
    assert np.all(z["v8"] == 0) and np.all(z["v_scale"] == 1.0)
    np.testing.assert_array_equal(z["v_mean"], oa.widen_bf16(v[0]).astype(np.float32))
    # q has no smoothing: every element is the block amax -> +448
    assert np.all(z["q8"] == 0x7E)
    np.testing.assert_allclose(z["q_scale"], 0.75 / 448, rtol=1e-7)


def test_block_means_closed_form():
    """Means of an arithmetic progression over each 64-token block (and the
    ragged last block of 150 - 128 = 22 tokens)."""
    S, D = 150, 128
    t = np.arange(S, dtype=np.float32)[:, None] * np.ones((1, D), np.float32)
    z = fp8.quantize_head(_bf16(t), _bf16(t), _bf16(t))
    np.testing.assert_array_equal(z["k_mean"][:, 0], [31.5, 95.5, (128 + 149) / 2])
    np.testing.assert_array_equal(z["v_mean"], np.full(D, 74.5, np.float32))
    zg = fp8.quantize_head(_bf16(t), _bf16(t), _bf16(t), k_mean="global")
    np.testing.assert_array_equal(zg["k_mean"], np.full((1, D), 74.5, np.float32))


def test_dequantisation_error_bound():
    """Relative half-ulp (2^-4) in the normal range, 2^-10 absolute (in scaled
    units) below it, and the block maximum lands on the top code."""
    g = np.random.default_rng(3)
    S, D = 300, 128
    q, k, v = (_bf16(g.standard_normal((S, D)) * s) for s in (1.0, 3.0, 2.0))
    z = fp8.quantize_head(q, k, v)
    blk = np.arange(S) // 64
    q32 = oa.widen_bf16(q)
    x = q32 / z["q_scale"][blk][:, None].astype(np.float64)  # scaled units, |x| <= ~448
    err = np.abs(x - fp8.e4m3_decode(z["q8"]))
    assert np.all(err <= np.maximum(2.0 ** -4 * np.abs(x), 2.0 ** -10) * (1 + 1e-6) + 1e-4)
    for b in range(blk.max() + 1):
        codes = z["q8"][blk == b]
        assert ((codes & 0x7F) == 0x7E).any()
    vres = oa.widen_bf16(v) - z["v_mean"].astype(np.float64)
    vh = fp8.e4m3_decode(z["v8"]) * z["v_scale"]
    assert np.all(np.abs(vres - vh) <= np.maximum(2.0 ** -4 * np.abs(vres), 2.0 ** -10 * z["v_scale"]) * 1.001 + 1e-6)


def test_blocks_are_independent():
    g = np.random.default_rng(4)
    S, D = 256, 128
    q, k, v = (_bf16(g.standard_normal((S, D))) for _ in range(3))
    k2 = k.copy()
    k2[140, 7] = _bf16(np.array([9.0]))[0]
    a, b = fp8.quantize_head(q, k, v), fp8.quantize_head(q, k2, v)
    changed = np.nonzero(a["k_scale"] != b["k_scale"])[0].tolist()
    assert changed == [2]
    assert np.array_equal(a["k8"][:128], b["k8"][:128]) and np.array_equal(a["k8"][192:], b["k8"][192:])


def _random_qz(S, D, seed, nb_mean):
    g = np.random.default_rng(seed)
    nb = -(-S // 64)
    finite = np.array([c for c in FINITE])
    return {
        "q8": g.choice(finite, (S, D)).astype(np.uint8),
        "k8": g.choice(finite, (S, D)).astype(np.uint8),
        "v8": g.choice(finite, (S, D)).astype(np.uint8),
        "q_scale": (g.uniform(0.5, 2, nb) / 448).astype(np.float32),
        "k_scale": (g.uniform(0.5, 2, nb) / 448).astype(np.float32),
        "k_mean": g.standard_normal((nb_mean, D)).astype(np.float32),
        "v_mean": g.standard_normal(D).astype(np.float32),
        "v_scale": (g.uniform(0.5, 2, D) / 448).astype(np.float32),
    }


@pytest.mark.parametrize("global_mean", [False, True])
def test_quant_model_without_p_quantisation_is_sdpa_on_dequantised(global_mean):
    """Library routine special case: with P unquantised, the model equals
    textbook attention (torch fp64 SDPA) on Q_hat, K_hat + k_mean, V_hat + v_mean."""
    torch = pytest.importorskip("torch")
    S, D = 200, 128
    nb = -(-S // 64)
    z = _random_qz(S, D, 5, 1 if global_mean else nb)
    blk = np.arange(S) // 64
    qh = fp8.e4m3_decode(z["q8"]) * z["q_scale"][blk][:, None].astype(np.float64)
    kh = fp8.e4m3_decode(z["k8"]) * z["k_scale"][blk][:, None].astype(np.float64)
    kh = kh + (z["k_mean"][0][None, :] if global_mean else z["k_mean"][blk]).astype(np.float64)
    vh = fp8.e4m3_decode(z["v8"]) * z["v_scale"][None, :].astype(np.float64) + z["v_mean"].astype(np.float64)
    scale = float(np.float32(0.088388))
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(np.ascontiguousarray(t))[None, None] for t in (qh, kh, vh)), scale=scale)[0, 0].numpy()
    got = fp8.attention_fp8_model_head(z, scale, p_quant=False)
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-11)


def test_quant_model_p_quantisation_bound():
    """Each quantised weight is within a relative 2^-4 of p in E4M3's normal
    range, so the normalised weights w/sum(w) and p/sum(p) differ by a factor
    within [(1 - 2^-4)/(1 + 2^-4), (1 + 2^-4)/(1 - 2^-4)] and
    |O_q - O| <= sum_j |w~_j - p~_j| max|V_hat| <= 0.134 max|V_hat| (weights in
    E4M3's subnormal range add at most S 2^-9/448 to the sum of differences)."""
    S, D = 130, 128
    z = _random_qz(S, D, 6, 3)
    scale = 0.05
    a = fp8.attention_fp8_model_head(z, scale, p_quant=True)
    b = fp8.attention_fp8_model_head(z, scale, p_quant=False)
    vmax = np.max(np.abs(fp8.e4m3_decode(z["v8"]) * z["v_scale"]))
    bound = ((1 + 2.0 ** -4) / (1 - 2.0 ** -4) - 1 + S * 2.0 ** -9 / 448) * vmax
    assert np.max(np.abs(a - b)) <= bound
    assert np.max(np.abs(a - b)) > 0


def test_quant_model_bruteforce_tiny():
    """Brute force in plain Python loops on a tiny head: scores, integer
    reference, E4M3 weights from the code table, weights normalised by their
    own sum, value mean added back."""
    S, D = 9, 128
    z = _random_qz(S, D, 21, 1)
    scale = 0.11
    got = fp8.attention_fp8_model_head(z, scale)
    table = fp8.e4m3_table()
    dec = lambda c: float(table[int(c)])
    log2e = 1.0 / math.log(2.0)
    for i in range(S):
        qi = [dec(z["q8"][i, d]) * float(z["q_scale"][0]) for d in range(D)]
        t = []
        for j in range(S):
            kj = [dec(z["k8"][j, d]) * float(z["k_scale"][0]) + float(z["k_mean"][0, d]) for d in range(D)]
            t.append(sum(a * b for a, b in zip(qi, kj)) * scale * log2e)
        m = math.ceil(max(t))
        w = []
        for j in range(S):
            p = 2.0 ** (t[j] - m)
            # nearest E4M3 value of 448 p (ties to the even code), from the table
            x = 448.0 * p
            best = min(range(127), key=lambda c: (abs(float(table[c]) - x), c & 1))
            w.append(float(table[best]) / 448.0)
        l = sum(w)
        for d in range(0, D, 37):
            o = sum(w[j] * dec(z["v8"][j, d]) * float(z["v_scale"][d]) for j in range(S)) / l
            assert abs(got[i, d] - (o + float(z["v_mean"][d]))) <= 1e-12 * (1 + abs(o))


def test_restore_returns_the_mean_for_constant_v():
    """V-Smooth restore (VC-Attention article, section 02): with a constant V
    the residual is zero and the output is the mean, exactly."""
    g = np.random.default_rng(8)
    S, D = 190, 128
    q = _bf16(g.standard_normal((S, D)))
    k = _bf16(g.standard_normal((S, D)) * 2)
    row = g.standard_normal(D)
    v = _bf16(np.tile(row, (S, 1)))
    z = fp8.quantize_head(q, k, v)
    out = fp8.attention_fp8_model_head(z, 1 / math.sqrt(D))
    np.testing.assert_array_equal(out, np.tile(oa.widen_bf16(v[0]), (S, 1)))


def test_v_smoothing_removes_offset_error():
    """Demean (VC-Attention article, section 02): with a large shared value
    offset the smoothed model is far closer to the truth than quantising V
    with its offset (emulated by a zero mean and the raw-V scale)."""
    g = np.random.default_rng(9)
    S, D = 256, 128
    q = _bf16(g.standard_normal((S, D)))
    k = _bf16(g.standard_normal((S, D)))
    v = _bf16(g.standard_normal((S, D)) + 20.0)
    scale = 1 / math.sqrt(D)
    truth = oa.attention_head(q, k, v, scale)
    z = fp8.quantize_head(q, k, v)
    smooth = fp8.attention_fp8_model_head(z, scale)
    raw = dict(z)
    v32 = oa.widen_bf16(v).astype(np.float32)
    amax = np.max(np.abs(v32), axis=0)
    raw["v_scale"] = (amax / np.float32(448)).astype(np.float32)
    raw["v8"] = fp8.e4m3_encode(np.clip(v32 * (np.float32(448) / amax), -448, 448))
    raw["v_mean"] = np.zeros(D, np.float32)
    unsmoothed = fp8.attention_fp8_model_head(raw, scale)
    assert fp8.max_abs(smooth, truth) * 4 < fp8.max_abs(unsmoothed, truth)


def test_k_block_mean_compensation_is_exact_without_quantisation_error():
    """With codes that represent K - k_mean exactly, the compensated scores are
    the scores of the original K (per-block mean: q.(k - m_b) + q.m_b)."""
    g = np.random.default_rng(10)
    S, D = 128, 128
    z = _random_qz(S, D, 11, 2)
    blk = np.arange(S) // 64
    kh = fp8.e4m3_decode(z["k8"]) * z["k_scale"][blk][:, None].astype(np.float64) + z["k_mean"][blk]
    qh = fp8.e4m3_decode(z["q8"]) * z["q_scale"][blk][:, None].astype(np.float64)
    vh = fp8.e4m3_decode(z["v8"]) * z["v_scale"][None, :].astype(np.float64)
    ref = oa.attention_head(qh, kh, vh, 0.07) + z["v_mean"]
    got = fp8.attention_fp8_model_head(z, 0.07, p_quant=False)
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-11)
    del g


def test_metrics():
    a = np.array([1.0, 2.0, 3.0])
    assert fp8.cosine(a, 2 * a) == pytest.approx(1.0)
    assert fp8.max_abs(a, a + [0, 0.5, 0]) == 0.5
    assert fp8.mean_rel_l1(a + [0.6, 0, 0], a) == pytest.approx(0.1)


# ---- ExpCast-FP8 (VC-Attention article, section 03) ----

def test_expcast_byte_is_log_affine_at_powers_of_two():
    """The E4M3 byte of 2^k, read as an integer, is exactly 8k + 56 (the
    format: exponent field k + 7, zero mantissa) over the normal range."""
    for k in range(-6, 9):
        assert int(fp8.e4m3_encode(np.array([2.0 ** k]))[0]) == 8 * k + 56


def test_expcast_matches_exact_cast_796_percent_per_octave():
    """The article's figures: per doubling of the value, the direct byte
    equals the exp-then-cast byte in 79.6% of cases and otherwise differs by
    one code."""
    u = (np.arange(200000) + 0.5) / 200000
    for k in (-5, -1, 0, 3, 7):
        v = 2.0 ** (u + k)
        exact = fp8.e4m3_encode(v).astype(np.int64)
        cast = fp8.expcast_byte(u + k).astype(np.int64)
        d = cast - exact
        assert abs(float(np.mean(d == 0)) - 0.796) < 0.0015, k
        assert int(np.max(np.abs(d))) == 1


def test_expcast_total_variation_bound():
    """The article's per-row bound: the ratio r of the ExpCast value to 2^t
    stays in [a, b] with (sqrt b - sqrt a)/(sqrt b + sqrt a) = 3.64%, the
    largest total variation such a ratio can cause between normalised
    weights; rows of scores without underflow stay under it."""
    table = fp8.e4m3_table()
    u = (np.arange(100000) + 0.5) / 100000 + 2
    r = table[fp8.expcast_byte(u)] / 2.0 ** u
    a, b = r.min(), r.max()
    bound = (math.sqrt(b) - math.sqrt(a)) / (math.sqrt(b) + math.sqrt(a))
    assert abs(bound - 0.0364) < 0.0005
    g = np.random.default_rng(12)
    for sd in (0.5, 1.0, 2.0):
        t = g.standard_normal(4096) * sd
        m = math.ceil(t.max())
        p = 2.0 ** (t - m)
        w = table[fp8.expcast_byte(t - m + math.log2(448))] / 448
        tv = 0.5 * np.abs(w / w.sum() - p / p.sum()).sum()
        assert tv < bound


def expcast_code_bruteforce(x):
    """ExpCast code of the byte position x, written out on the E4M3 grids:
    a position at or above 7.5 is its own byte (round half to even); below,
    the byte map's value 2^(floor(x/8) - 7) (1 + (x/8 - floor(x/8))) is put
    on the subnormal grid of steps 2^-9 (round half to even), where code c
    is c 2^-9 (and 8 2^-9 = 2^-6 is the first normal code, byte 8)."""
    if x == -math.inf:
        return 0
    if x >= 7.5:
        return int(round_half_even(x))
    e = math.floor(x / 8)
    val = 2.0 ** (e - 7) * (1 + (x / 8 - e))
    return int(round_half_even(val * 512))


def test_expcast_model_uses_the_direct_bytes():
    """Model with p_cast='expcast' = the textbook weighted mean with the
    ExpCast weights, written out for a tiny head whose rows reach the
    subnormal codes."""
    S, D = 40, 128
    z = _random_qz(S, D, 22, 1)
    scale = 2.0
    got = fp8.attention_fp8_model_head(z, scale, p_cast="expcast")
    table = fp8.e4m3_table()
    qh = fp8.e4m3_decode(z["q8"]) * float(z["q_scale"][0])
    kh = fp8.e4m3_decode(z["k8"]) * float(z["k_scale"][0]) + z["k_mean"][0].astype(np.float64)
    vh = fp8.e4m3_decode(z["v8"]) * z["v_scale"].astype(np.float64)
    t = (qh @ kh.T) * scale / math.log(2.0)
    n_sub = 0
    for i in range(S):
        m = math.ceil(t[i].max())
        x = 8 * (t[i] - m) + 8 * math.log2(448) + 56 - 0.35
        codes = [expcast_code_bruteforce(float(xx)) for xx in x]
        n_sub += sum(0 < c < 8 for c in codes)
        w = np.array([table[c] for c in codes])
        o = (w @ vh) / w.sum() + z["v_mean"]
        np.testing.assert_allclose(got[i], o, rtol=1e-12, atol=1e-12)
    assert n_sub > 20   # the case exercises the subnormal codes


def round_half_even(x):
    r = math.floor(x + 0.5)
    if r - x == 0.5 and r % 2 == 1:
        r -= 1
    return r


def test_expcast_within_one_code_of_the_exact_cast():
    """The article's accuracy claim, "otherwise one code off", over the whole
    range a weight 448 p can take down to where the exact cast reaches zero:
    log2 v in [-9.5, log2 448], subnormal codes included."""
    u = np.linspace(-9.5, math.log2(448), 1_000_001)
    d = fp8.expcast_byte(u).astype(np.int64) - fp8.e4m3_encode(2.0 ** u).astype(np.int64)
    assert int(np.max(np.abs(d))) == 1
    sub = u < -6
    assert np.mean(d[sub] == 0) > 0.5


def test_expcast_subnormal_codes_at_known_points():
    """Closed-form points below the normal range: position x = 8 log2 v +
    55.65; x = 0 gives 2^-7 (1 + 0) -> code 4 (4 2^-9); x = -8 gives 2^-8 ->
    code 2; x = -16 gives 2^-9 -> code 1; x = -24 gives 2^-10 = half a step,
    a tie -> code 0 (even); x = 6 gives 2^-7 (1 + 6/8) = 7 2^-9 -> code 7;
    x = 7.4 gives 2^-7 (1 + 0.925) = 7.7 2^-9 -> code 8."""
    for x, code in ((0.0, 4), (-8.0, 2), (-16.0, 1), (-24.0, 0), (6.0, 7), (7.4, 8), (-40.0, 0)):
        u = (x - 56 + 0.35) / 8
        assert int(fp8.expcast_byte(np.array([u]))[0]) == code, x
        assert expcast_code_bruteforce(x) == code, x
    assert int(fp8.expcast_byte(np.array([-np.inf]))[0]) == 0


def test_expcast_weights_commute_with_powers_of_two_in_the_normal_range():
    """Shifting log2 v by an integer k shifts the byte by 8 k and multiplies
    the decoded weight by exactly 2^k while both stay normal: an online
    softmax whose reference rises by whole powers of two writes the same
    weights as one taken against the final row maximum."""
    g = np.random.default_rng(31)
    u = g.uniform(-5.5, 0.0, 200000)
    table = fp8.e4m3_table()
    base = fp8.expcast_byte(u).astype(np.int64)
    for k in (1, 2, 5, 8):
        shifted = fp8.expcast_byte(u + k).astype(np.int64)
        np.testing.assert_array_equal(shifted, base + 8 * k)
        np.testing.assert_array_equal(table[shifted], table[base] * 2.0 ** k)


@pytest.mark.parametrize("p_cast", ["exp", "expcast"])
def test_model_invariant_to_joint_block_permutation(p_cast):
    """The same permutation of the keys' and values' 64-token blocks (codes,
    K scales and K means together) leaves every output row unchanged, for
    both casts (non-causal attention is a sum over keys; VC-Attention
    article, section 02, Group)."""
    S, D = 64 * 9, 128
    nb = S // 64
    z = _random_qz(S, D, 25, nb)
    perm = np.random.default_rng(3).permutation(nb)
    tok = (perm[:, None] * 64 + np.arange(64)[None, :]).ravel()
    zp = dict(z)
    zp["k8"], zp["v8"] = z["k8"][tok], z["v8"][tok]
    zp["k_scale"], zp["k_mean"] = z["k_scale"][perm], z["k_mean"][perm]
    # the queries keep their own blocks: q_scale is indexed by the query's
    # block, which does not move
    for scale in (0.1, 0.6):
        a = fp8.attention_fp8_model_head(z, scale, p_cast=p_cast)
        b = fp8.attention_fp8_model_head(zp, scale, p_cast=p_cast)
        np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("mask", ["causal", "sparse"])
def test_masked_model_without_p_quantisation_is_masked_attention(mask):
    """With P unquantised, the masked model is the masked definition on the
    dequantised operands; with quantisation every weight of a masked key is 0
    (exp and ExpCast)."""
    g = np.random.default_rng(11)
    S, D = 300, 128
    nb = -(-S // 64)
    z = _random_qz(S, D, 12, nb)
    if mask == "causal":
        allowed = oa.block_causal_allowed(S, 70)
    else:
        m = g.random((-(-S // 128), nb)) < 0.4
        m[:, 0] = True
        allowed = oa.tile_mask_allowed(S, 128, 64, m)
    blk = np.arange(S) // 64
    qh = fp8.e4m3_decode(z["q8"]) * z["q_scale"][blk][:, None].astype(np.float64)
    kh = fp8.e4m3_decode(z["k8"]) * z["k_scale"][blk][:, None].astype(np.float64) + z["k_mean"][blk]
    vh = fp8.e4m3_decode(z["v8"]) * z["v_scale"][None, :].astype(np.float64) + z["v_mean"]
    scale = 0.07
    ref = oa.attention_head(qh, kh, vh, scale, allowed=allowed)
    got = fp8.attention_fp8_model_head(z, scale, p_quant=False, allowed=allowed)
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-11)
    # quantised weights: permuting the values of the keys row 0 may not see
    # changes nothing in row 0
    hidden = np.flatnonzero(~allowed(np.arange(1))[0])
    assert hidden.size > 10
    z2 = dict(z)
    v2 = z["v8"].copy()
    v2[hidden] = v2[hidden[::-1]]
    z2["v8"] = v2
    for p_cast in ("exp", "expcast"):
        kw = dict(p_cast=p_cast, allowed=allowed)
        a = fp8.attention_fp8_model_head(z, scale, **kw)
        b = fp8.attention_fp8_model_head(z2, scale, **kw)
        assert np.all(np.isfinite(a))
        np.testing.assert_array_equal(a[0], b[0])
