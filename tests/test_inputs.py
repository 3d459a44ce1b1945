"""The seeded generator: determinism, prefix property and workload structure."""

import numpy as np

from video_diffusion_transformer_vdit_amd import inputs


def test_same_seed_same_bytes():
    w = inputs.get_workload("tiny-3x16x16")
    a = inputs.make_inputs(w, threads=1)
    b = inputs.make_inputs(w, threads=4)
    for x, y in zip(a, b):
        assert x.dtype == np.uint16 and x.shape == w.shape
        assert np.array_equal(x, y)
    assert not np.array_equal(a[0], a[1])


def test_shorter_plane_is_prefix():
    w = inputs.get_workload("wan2.1-14b-720p")
    full = inputs.make_plane(w, "k", 0, 3, S=1000)
    assert np.array_equal(inputs.make_plane(w, "k", 0, 3, S=137), full[:137])


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 3.14159], np.float32)
    bits = inputs.f32_to_bf16_bits(x)
    back = inputs.bf16_bits_to_f32(bits)
    # ulp at 1 is 2^-7: 1 + 2^-8 ties to 1.0 (even); 1 + 3*2^-8 ties to 1 + 2*2^-7 (even)
    assert back.tolist()[:5] == [1.0, 1.0, 1.0 + 4 * 2 ** -8, 1.0, -2.5]
    assert abs(back[5] - 3.14159) < 2 ** -7 * 4


def test_outlier_structure():
    w = inputs.get_workload("wan2.1-14b-720p")
    S = 4000
    ch = inputs.outlier_channels(w, 5)
    assert len(set(ch.tolist())) == 4
    for t in ("k", "v"):
        x = inputs.bf16_bits_to_f32(inputs.make_plane(w, t, 0, 5, S=S))
        std = x.std(axis=0)
        assert np.all(std[ch] > 6) and np.all(np.delete(std, ch) < 1.2)
    q = inputs.bf16_bits_to_f32(inputs.make_plane(w, "q", 0, 5, S=S))
    assert np.all(q.std(axis=0) < 1.2)


def test_k_offset_structure():
    w = inputs.get_workload("wan2.1-1.3b-480p")
    k = inputs.bf16_bits_to_f32(inputs.make_plane(w, "k", 0, 2, S=20000)).astype(np.float64)
    off = inputs.k_offsets(w, 2)
    assert np.max(np.abs(k.mean(axis=0) - off)) < 0.05
    assert 0.3 < off.std() < 0.7


def test_workload_table():
    names = set(inputs.WORKLOADS)
    assert {"tiny-3x16x16", "wan2.1-1.3b-480p", "wan2.2-720p-16x", "wan2.1-14b-720p",
            "wan2.1-14b-720p-fp8"} <= names
    for w in inputs.WORKLOADS.values():
        assert w.S == w.frames * w.tokens_per_frame and w.D == 128


def test_block_mask_recipe():
    m = inputs.make_block_mask(1, 2, 1000, 0.25, seed=3)
    assert m.shape == (1, 2, 8, 16) and m.dtype == np.uint8
    # row blocks of one 256-query group share their selection
    assert np.array_equal(m[:, :, 0::2], m[:, :, 1::2])
    # every row block keeps its own key tiles and at least a quarter overall
    for qb in range(8):
        own = slice(qb * 2, min(16, qb * 2 + 2))
        assert np.all(m[:, :, qb, own] == 1)
    assert np.all(m.sum(axis=3) >= 4)
    # seeded
    assert np.array_equal(m, inputs.make_block_mask(1, 2, 1000, 0.25, seed=3))
