"""Pins for the oracle's structured rotation Pi = H D / sqrt(d) (CPU only).

ai-coding.wiselychen.com, "Google TurboQuant：KV Cache 壓縮 6x…", community
implementation section (TurboQuant+): a Walsh-Hadamard rotation in place of
the dense one, with the rotated coordinates near Gaussian (kurtosis about 900
before, about 2.9 after).  The Hadamard matrix is checked against its
recursive definition, the rotation against an independent butterfly
transform, the signs against the stream's top bits, and the method's
behaviour (Gaussianisation, MSE distortion, unbiased inner products) against
the same closed forms and page values as the dense rotation.
"""
import math

import numpy as np
import pytest

from oracle import tq_oracle as o


def _sylvester(d):
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


@pytest.mark.parametrize("d", [1, 2, 4, 8, 64, 128, 256])
def test_hadamard_is_the_sylvester_recursion(d):
    assert np.array_equal(o.hadamard(d), _sylvester(d))


def test_hadamard_rejects_other_orders():
    with pytest.raises(ValueError):
        o.hadamard(96)


@pytest.mark.parametrize("d", [4, 64, 128, 256])
def test_hadamard_rotation_orthogonal(d):
    pi = o.rotation_hadamard(d, 5)
    assert np.max(np.abs(pi @ pi.T - np.eye(d))) < 1e-13
    assert np.allclose(np.abs(pi), 1 / math.sqrt(d), rtol=0, atol=1e-16)


def _fwht(x):
    """In-place butterfly Walsh-Hadamard transform along the last axis."""
    x = x.copy()
    n = x.shape[-1]
    h = 1
    while h < n:
        x = x.reshape(*x.shape[:-1], n // (2 * h), 2, h)
        a, b = x[..., 0, :].copy(), x[..., 1, :].copy()
        x[..., 0, :], x[..., 1, :] = a + b, a - b
        x = x.reshape(*x.shape[:-3], n)
        h *= 2
    return x


@pytest.mark.parametrize("d", [8, 128, 256])
def test_rotation_equals_butterfly_transform(d):
    rng = np.random.default_rng(d)
    x = rng.standard_normal((20, d))
    s = o.rademacher_signs(3, d)
    fast = _fwht(x * s[None, :]) / math.sqrt(d)
    assert np.max(np.abs(fast - x @ o.rotation_hadamard(d, 3).T)) < 1e-12


def test_signs_are_the_stream_top_bits():
    d = 4096
    s = o.rademacher_signs(11, d)
    z = o.splitmix64(o.stream_state(11, o.TAG_SIGNS), d)
    assert np.array_equal(s < 0, z >= np.uint64(1 << 63))
    assert abs(s.mean()) < 4 / math.sqrt(d)
    # a stream of its own: not the rotation's or the QJL matrix's top bits
    for tag in (o.TAG_ROTATION, o.TAG_QJL):
        zt = o.splitmix64(o.stream_state(11, tag), d)
        assert not np.array_equal(s < 0, zt >= np.uint64(1 << 63))


def test_hadamard_gaussianises_heavy_tailed_coordinates(golden):
    # Student-t (5 dof) coordinates, kurtosis about 9: after H D / sqrt(d)
    # every rotated coordinate mixes all d inputs with equal weight, and the
    # pooled kurtosis lands near the Gaussian value 3 d / (d + 2) of a unit
    # vector's coordinate (the page: near-Gaussian after rotation, 2.9)
    pv = golden["pages"]["kurtosis_after_rotation"]
    d, n = 128, 20000
    x = np.random.default_rng(2).standard_t(5, (n, d))
    before = np.mean(x ** 4) / np.mean(x ** 2) ** 2
    u = x / np.linalg.norm(x, axis=1, keepdims=True)
    y = u @ o.rotation_hadamard(d, 0).T
    after = np.mean(y ** 4) / np.mean(y ** 2) ** 2
    assert before > 6
    assert abs(after - 3 * d / (d + 2)) < 0.1 and abs(after - pv["after"]) < 0.15


def test_hadamard_on_fixed_outlier_channels_is_platykurtic():
    # Documented difference from the dense rotation: with 4 fixed channels
    # scaled x20, every rotated coordinate is (+-u_a +-u_b +-u_c +-u_d)/sqrt(d)
    # plus a small Gaussian part, i.e. close to one coordinate of a point on
    # the 3-sphere (kurtosis 3*4/(4+2) = 2), while a Haar rotation mixes the
    # channels with random weights per coordinate and lands near 3.
    d, n = 128, 20000
    rng = np.random.default_rng(1)
    x = rng.standard_normal((n, d))
    x[:, rng.choice(d, 4, replace=False)] *= 20.0
    u = x / np.linalg.norm(x, axis=1, keepdims=True)
    k_h = [np.mean(y ** 4) / np.mean(y ** 2) ** 2 for y in [u @ o.rotation_hadamard(d, s).T for s in (0, 1)]]
    y = u @ o.rotation(d, 0).T
    k_haar = np.mean(y ** 4) / np.mean(y ** 2) ** 2
    assert all(2.0 < k < 2.4 for k in k_h)
    assert abs(k_haar - 3 * d / (d + 2)) < 0.1


@pytest.mark.parametrize("bp", [1, 2, 3, 4])
def test_mse_distortion_matches_the_beta_law_value(bp):
    # Gaussian vectors are rotation invariant in law, so after H D / sqrt(d)
    # the unit vector's coordinates follow the same Beta law as after a Haar
    # rotation: the Monte Carlo distortion meets the analytic value.
    d, n = 128, 60000
    qz = o.Quantizer(d, bp, seed=0, rotation_kind="hadamard")
    rng = np.random.default_rng(bp + 10)
    u = rng.standard_normal((n, d))
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    idx, nrm = o.encode_mse(qz, u)
    err = np.sum((u - o.decode_mse(qz, idx, nrm)) ** 2, axis=1)
    c, t = o.lloyd_max(d, 2 ** bp)
    D = o.codebook_distortion(d, c, t)
    assert abs(err.mean() - D) < 3 * err.std() / math.sqrt(n)


def test_inner_product_estimate_unbiased_with_hadamard_rotation():
    # logit = <q, decode_prod(x)> holds for any orthogonal Pi, and its mean
    # over QJL draws equals <q, x> (the dense-rotation test's experiment)
    d, trials = 64, 3000
    rng = np.random.default_rng(4)
    x = rng.standard_normal((1, d))
    q = rng.standard_normal((1, d))
    est = []
    for seed in range(trials):
        qz = o.Quantizer(d, 2, seed=seed, rotation_kind="hadamard")
        idx, bits, n, g = o.encode_prod(qz, x)
        est.append(o.scores(qz, q, idx, bits, n, g)[0, 0])
        if seed < 3:
            ref = (q @ o.decode_prod(qz, idx, bits, n, g).T)[0, 0]
            assert abs(est[-1] - ref) < 1e-10 * abs(ref) + 1e-12
    est = np.array(est)
    true = float(q @ x.T)
    assert abs(est.mean() - true) < 4 * est.std() / math.sqrt(trials)
