"""Pins for the V-Smooth Group checker (k-means of value tokens and the joint
K/V permutation; VC-Attention article, section 02).  CPU only."""

import math

import numpy as np
import pytest

from oracle import attention as oa
from oracle import group


def test_assignment_is_the_nearest_centroid_by_direct_distance():
    g = np.random.default_rng(1)
    v = g.standard_normal((500, 16))
    mu = g.standard_normal((23, 16))
    direct = np.array([min(range(23), key=lambda c: math.fsum((v[i] - mu[c]) ** 2)) for i in range(500)])
    np.testing.assert_array_equal(group.assign(v, mu), direct)


def test_ties_go_to_the_lowest_cluster():
    v = np.array([[0.0, 0.0], [1.0, 0.0]])
    mu = np.array([[1.0, 1.0], [1.0, -1.0], [-1.0, 1.0]])  # token 0 equidistant to all three
    assert group.assign(v, mu)[0] == 0


def test_update_is_the_member_mean_and_empty_clusters_stay():
    g = np.random.default_rng(2)
    v = g.standard_normal((300, 8))
    labels = g.integers(0, 6, 300)
    labels[labels == 4] = 5  # cluster 4 empty
    mu0 = g.standard_normal((6, 8))
    new = group.update(v, labels, mu0)
    for c in range(6):
        members = [v[i] for i in range(300) if labels[i] == c]
        want = mu0[c] if not members else np.array([math.fsum(col) / len(members) for col in zip(*members)])
        np.testing.assert_allclose(new[c], want, rtol=1e-13, atol=1e-13)


def test_lloyd_rounds_never_increase_the_objective():
    g = np.random.default_rng(3)
    v = g.standard_normal((2000, 32)) + 3 * g.standard_normal((20, 32))[g.integers(0, 20, 2000)]
    mu = group.initial_centroids(v, 16)
    prev = math.inf
    for _ in range(6):
        lab = group.assign(v, mu)
        obj = group.objective(v, lab, mu)
        assert obj <= prev * (1 + 1e-12)
        prev = obj
        mu = group.update(v, lab, mu)
        assert group.objective(v, lab, mu) <= obj * (1 + 1e-12)


def test_exact_points_are_a_fixed_point():
    """Tokens that are copies of k distinct points, arranged so that the start
    picks each point once: one round changes nothing and the permutation
    groups identical tokens, in token order."""
    g = np.random.default_rng(4)
    k, S = 8, 800
    pts = g.standard_normal((k, 16)) * 5
    lab_true = g.integers(0, k, S)
    starts = (np.arange(k) * S) // k
    lab_true[starts] = np.arange(k)
    v = pts[lab_true]
    labels, mu = group.kmeans_head(v, k, rounds=3)
    np.testing.assert_array_equal(labels, lab_true)
    np.testing.assert_allclose(mu, pts, rtol=1e-13, atol=1e-13)
    perm = group.stable_permutation(labels)
    assert perm.tolist() == sorted(range(S), key=lambda i: (lab_true[i], i))


def test_permutation_is_stable_sort_by_cluster():
    g = np.random.default_rng(5)
    labels = g.integers(0, 40, 3000)
    perm = group.stable_permutation(labels)
    assert perm.tolist() == sorted(range(3000), key=lambda i: (labels[i], i))


def test_joint_kv_permutation_leaves_attention_unchanged():
    g = np.random.default_rng(6)
    q, k, v = (g.standard_normal((200, 128)) for _ in range(3))
    labels, _ = group.kmeans_head(v, 2)
    perm = group.stable_permutation(labels)
    a = oa.attention_head(q, k, v, 0.09)
    b = oa.attention_head(q, k[perm], v[perm], 0.09)
    np.testing.assert_allclose(b, a, rtol=1e-12, atol=1e-13)


def test_grouping_raises_the_energy_block_means_remove():
    """Clustered values in random order: block means of the sequence order
    remove little; after grouping they remove most of the cluster part (the
    article's 8% -> 36% direction)."""
    g = np.random.default_rng(7)
    S, D = 128 * 40, 128
    centers = g.standard_normal((40, D)) * 2
    v = centers[g.integers(0, 40, S)] + g.standard_normal((S, D))
    before = group.block_energy_removed(v)
    labels, _ = group.kmeans_head(v, 40, rounds=4)
    after = group.block_energy_removed(v, group.stable_permutation(labels))
    assert before < 0.05 and after > 0.5, (before, after)


def test_block_energy_closed_form():
    """Blocks that are constant vectors lose all their energy; zero-mean
    blocks lose none."""
    c = np.repeat(np.arange(1.0, 5.0)[:, None], 128, axis=0) * np.ones((1, 4))
    assert group.block_energy_removed(c) == pytest.approx(1.0, rel=1e-15)
    z = np.tile(np.array([[1.0], [-1.0]]), (256, 3))
    assert group.block_energy_removed(z) == 0.0
