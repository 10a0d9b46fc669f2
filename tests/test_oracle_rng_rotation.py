"""Pins for the oracle's seeded generator and the rotation / sketch matrices."""
import numpy as np
import pytest
from scipy import stats

from oracle import rng, rotation
from tests.conftest import load_golden


def test_splitmix64_published_vector():
    g = load_golden("splitmix64_seed0.json")
    out = rng.splitmix64(g["seed"], 3)
    assert [int(v) for v in out] == [int(h, 16) for h in g["outputs_hex"]]


def test_splitmix64_counter_form_matches_sequential_bigint():
    # Sequential state updates with Python integers (the generator's stepwise
    # definition) against the counter form used by the oracle.
    m = (1 << 64) - 1
    seed = 42 + 7 * 5
    state = seed
    ref = []
    for _ in range(50):
        state = (state + 0x9E3779B97F4A7C15) & m
        z = state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & m
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & m
        ref.append(z ^ (z >> 31))
    got = rng.splitmix64(seed, 50)
    assert [int(v) for v in got] == ref
    # A window deep in the stream equals the same outputs drawn from the start.
    assert np.array_equal(rng.splitmix64(seed, 10, start=40), got[40:50])


def test_uniform_and_normal_laws():
    u = rng.uniforms(7, 200000)
    assert u.min() > 0.0 and u.max() < 1.0
    assert stats.kstest(u, "uniform").pvalue > 1e-3
    z = rng.normals(7, 200000)
    assert stats.kstest(z, "norm").pvalue > 1e-3
    assert abs(z.mean()) < 4.5 / np.sqrt(len(z))
    assert abs(z.var() - 1.0) < 4.5 * np.sqrt(2.0 / len(z))


def test_layer_seed_from_page():
    g = load_golden("page_constants.json")["layer_seed"]
    for layer, seed in g["examples"].items():
        assert rng.layer_seed(int(layer)) == seed


@pytest.mark.parametrize("d", [8, 32, 128])
def test_rotation_is_orthogonal_with_positive_r(d):
    seed = 42
    g, _ = rotation.gaussian_matrices(d, seed)
    pi64, _ = rotation.make_rotations(d, seed, as_stored=False)
    assert np.max(np.abs(pi64.T @ pi64 - np.eye(d))) < 1e-12
    # G = Pi R with R upper triangular and a positive diagonal (the unique QR
    # that makes Pi Haar distributed).
    r = pi64.T @ g
    assert np.max(np.abs(np.tril(r, -1))) < 1e-10 * np.max(np.abs(r))
    assert np.all(np.diag(r) > 0)
    pi32, s32 = rotation.make_rotations(d, seed, as_stored=True)
    assert np.max(np.abs(pi32.T @ pi32 - np.eye(d))) < 1e-6
    assert np.array_equal(pi32, pi64.astype(np.float32).astype(np.float64))


def test_rotation_storage_size_from_page():
    c = load_golden("page_constants.json")["rotation_bytes"]
    pi, _ = rotation.make_rotations(c["d"], 42)
    assert pi.astype(np.float32).nbytes == c["bytes"]


def test_rotated_coordinates_follow_the_beta_law():
    # Haar rotation of a fixed unit vector: each coordinate follows f_d, i.e.
    # (t+1)/2 ~ Beta((d-1)/2, (d-1)/2).  Pool the first coordinate over many
    # independent rotations.
    d = 16
    e = np.zeros(d)
    e[0] = 1.0
    ys = np.array([rotation.make_rotations(d, 1000 + i, as_stored=False)[0] @ e
                   for i in range(3000)])
    a = (d - 1) / 2
    for j in (0, 5):
        assert stats.kstest((ys[:, j] + 1) / 2, stats.beta(a, a).cdf).pvalue > 1e-3


def test_sketch_is_standard_gaussian_and_distinct_from_rotation_stream():
    d = 128
    g, s = rotation.gaussian_matrices(d, 42)
    assert stats.kstest(s.ravel(), "norm").pvalue > 1e-3
    assert not np.allclose(g, s)
    _, s32 = rotation.make_rotations(d, 42)
    assert np.array_equal(s32, s.astype(np.float32).astype(np.float64))
