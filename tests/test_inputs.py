"""The seeded input generator: determinism, published test vector, moments (CPU)."""

import numpy as np
import pytest

from iterative_stencil_pde_amd import inputs


def test_splitmix64_published_vector():
    # SplitMix64 from state 0 yields 0xE220A8397B1DCDAF first (Steele, Lea, Flood 2014;
    # the same value Vigna's reference splitmix64.c prints). Key 0 is seed 0, stream 0, k 0.
    u = inputs.uniform(0, 0, 1)[0]
    assert u == (0xE220A8397B1DCDAF >> 11) * 2.0 ** -53


def test_same_seed_same_bytes_and_independent_streams():
    a = inputs.uniform(7, 1, 1000, -1, 1)
    b = inputs.uniform(7, 1, 1000, -1, 1)
    c = inputs.uniform(7, 2, 1000, -1, 1)
    d = inputs.uniform(8, 1, 1000, -1, 1)
    assert np.array_equal(a, b)
    assert not np.array_equal(a, c) and not np.array_equal(a, d)
    # counter-based: a prefix is a prefix
    assert np.array_equal(inputs.uniform(7, 1, 10, -1, 1), a[:10])


def test_uniform_moments():
    n = 200_000
    u = inputs.uniform(3, 0, n, 0.0, 1.0)
    assert u.min() >= 0.0 and u.max() < 1.0
    assert abs(u.mean() - 0.5) < 5 * np.sqrt(1 / 12 / n)
    assert abs(u.var() - 1 / 12) < 0.003
    v = inputs.uniform(2, 0, n, -1.0, 1.0)
    assert abs(v.mean()) < 5 * np.sqrt(1 / 3 / n) and abs(v.std() - 1 / np.sqrt(3)) < 0.003


def test_normal_moments():
    n = 200_000
    z = inputs.normal(5, 2, n, 0.0, 0.01)
    assert abs(z.mean()) < 5 * 0.01 / np.sqrt(n)
    assert abs(z.std() - 0.01) < 0.01 * 0.01
    # tails of a normal, not of a uniform
    assert 0.0025 < np.mean(np.abs(z) > 0.03) < 0.0030 + 0.0008


def test_sinpi_samples():
    s = inputs.sinpi_samples(65, 1 / 64, 1.0)
    assert s[0] == 0.0 and abs(s[-1]) < 1e-15 and s[32] == 1.0


@pytest.mark.parametrize("name", ["laplace64", "poisson256", "laplace1024"])
def test_workloads_shape_and_determinism(name):
    w1 = inputs.make(name)
    w2 = inputs.make(name)
    assert w1.digest() == w2.digest()
    assert w1.u0.shape == (w1.ny, w1.nx) and w1.u0.dtype == w1.dtype
    if w1.f is not None:
        assert w1.f.shape == w1.u0.shape and w1.f.dtype == w1.dtype


def test_workload_recipes():
    w = inputs.make("laplace64")
    assert w.sweeps == 1000 and w.f is None and w.h == 1 / 63
    x = np.arange(64) / 63
    assert np.array_equal(w.u0[0, :], (x * x - 0.0).astype(np.float32))
    assert np.all(w.u0[1:-1, 1:-1] == 0)
    assert np.array_equal(w.u0, -w.u0.T)
    w = inputs.make("poisson256")
    assert w.sweeps == 10000 and w.h == 1 / 255
    assert w.residual_checkpoints == list(range(0, 10001, 100))
    assert np.all(w.u0 == 0) and w.f.min() >= -1 and w.f.max() <= 1
    w = inputs.make("laplace1024")
    assert w.residual_checkpoints == list(range(0, 5001, 500))
    assert w.readback_checkpoints == list(range(0, 5001, 500))
    assert np.all(w.u0[0] == 0) and np.all(w.u0[:, -1] == 0) and w.u0[1:-1, 1:-1].min() >= 0
    w = inputs.laplace_top_edge(64, 10)
    assert np.all(w.u0[-1] == 1) and np.all(w.u0[:-1] == 0)
    w = inputs.poisson_sine_noise(65, 10, 5)
    assert w.dtype == np.float64 and w.h == 1 / 64
    assert w.residual_checkpoints == [0, 5, 10]
    s = np.sin(np.pi * np.arange(65) / 64)
    assert (w.f - s[:, None] * s[None, :]).std() == pytest.approx(0.01, rel=0.1)
