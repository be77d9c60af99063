"""Pins for the oracle's encode / decode / scores / layout (CPU only).

Encode: normalise, rotate, nearest centroid per coordinate, residual, QJL
signs and residual norm (blog.hotdry.top, both stage sections; a2a-mcp.org,
stage 1 and 2).  The nearest-centroid step is pinned by brute force over the
whole product codebook, the distortion by Monte Carlo against the analytic
value, the inner-product estimator by an unbiasedness experiment with a
negative control, and its variance by the closed form for Gaussian rows.
"""
import itertools
import math

import numpy as np
import pytest

from oracle import tq_oracle as o


def _unit(rng, n, d):
    u = rng.standard_normal((n, d))
    return u / np.linalg.norm(u, axis=1, keepdims=True)


@pytest.mark.parametrize("d,bits", [(3, 2), (3, 3), (4, 2), (4, 3)])
def test_bucketize_is_product_codebook_nearest(d, bits):
    # Brute force: the nearest of all K^d codewords of the product codebook to
    # y equals the per-coordinate threshold count.
    qz = o.Quantizer(d, bits, seed=5)
    bp, c, _ = qz.codebook("prod")
    K = 2 ** bp
    words = np.array(list(itertools.product(range(K), repeat=d)))     # [K^d, d]
    cw = c[words]
    rng = np.random.default_rng(0)
    x = rng.standard_normal((300, d)) * rng.uniform(0.1, 5, (300, 1))
    idx, _, n, _ = o.encode_prod(qz, x)
    y = (x / n[:, None]) @ qz.pi.T
    dist = ((y[:, None, :] - cw[None]) ** 2).sum(-1)
    best = words[np.argmin(dist, axis=1)]
    assert np.array_equal(best, idx)


def test_bucketize_is_per_coordinate_argmin():
    c, t = o.lloyd_max(128, 16)
    y = np.random.default_rng(1).normal(0, 1 / math.sqrt(128), 100000)
    assert np.array_equal(o.bucketize(y, t), np.argmin(np.abs(y[:, None] - c[None]), axis=1))


def test_threshold_ties_go_low():
    c, t = o.lloyd_max(128, 4)
    y = np.array([t[0], t[1], t[2], np.nextafter(t[1], 1)])
    assert list(o.bucketize(y, t)) == [0, 1, 2, 2]


@pytest.mark.parametrize("bp", [1, 2, 3, 4])
def test_monte_carlo_distortion(bp):
    d, n = 128, 100000
    qz = o.Quantizer(d, bp, seed=0)
    u = _unit(np.random.default_rng(bp), n, d)
    idx, nrm = o.encode_mse(qz, u)
    err = np.sum((u - o.decode_mse(qz, idx, nrm)) ** 2, axis=1)
    c, t = o.lloyd_max(d, 2 ** bp)
    D = o.codebook_distortion(d, c, t)
    assert abs(err.mean() - D) < 3 * err.std() / math.sqrt(n)


def test_encode_is_scale_invariant_and_norm_exact():
    qz = o.Quantizer(32, 3, seed=2)
    x = np.random.default_rng(3).standard_normal((50, 32))
    i1, b1, n1, g1 = o.encode_prod(qz, x)
    i2, b2, n2, g2 = o.encode_prod(qz, 7.5 * x)
    assert np.array_equal(i1, i2) and np.array_equal(b1, b2)
    assert np.allclose(n2, 7.5 * n1, rtol=1e-14) and np.allclose(g2, 7.5 * g1, rtol=1e-12)
    assert np.allclose(n1, np.sqrt((x ** 2).sum(1)), rtol=1e-14)


def test_gamma_is_residual_norm():
    qz = o.Quantizer(64, 3, seed=4)
    x = np.random.default_rng(4).standard_normal((20, 64))
    idx, bits, n, g = o.encode_prod(qz, x)
    r = x - o.mse_reconstruct(qz, "prod", idx, n)
    assert np.allclose(g, np.linalg.norm(r, axis=1), rtol=1e-13)
    # the residual in the rotated frame has the same norm (Pi orthogonal)
    y = (x / n[:, None]) @ qz.pi.T
    _, c, _ = qz.codebook("prod")
    assert np.allclose(g, n * np.linalg.norm(y - c[idx], axis=1), rtol=1e-12)
    assert np.array_equal(bits, (r @ qz.s.T >= 0).astype(np.uint8))


def test_zero_vector():
    qz = o.Quantizer(16, 3, seed=0)
    idx, bits, n, g = o.encode_prod(qz, np.zeros((1, 16)))
    K = 2 ** qz.bp_prod
    assert np.all(idx == K // 2 - 1) and np.all(bits == 1) and n[0] == 0 and g[0] == 0
    assert np.all(o.decode_prod(qz, idx, bits, n, g) == 0)
    assert np.all(o.scores(qz, np.ones((2, 16)), idx, bits, n, g) == 0)


def test_scores_equal_dot_with_decoded():
    # two routes: rotated-domain score from indices vs <q, decode(code)>
    qz = o.Quantizer(48, 3, seed=1)
    rng = np.random.default_rng(5)
    x = rng.standard_normal((64, 48)) * rng.uniform(0.5, 20, 48)
    q = rng.standard_normal((5, 48))
    idx, bits, n, g = o.encode_prod(qz, x)
    s1 = o.scores(qz, q, idx, bits, n, g)
    s2 = q @ o.decode_prod(qz, idx, bits, n, g).T
    assert np.max(np.abs(s1 - s2)) < 1e-10 * np.abs(s2).max()


def _tq_error_batch(qz, x, q, S):
    qz.s = S
    qz.m = S.shape[0]
    idx, bits, n, g = o.encode_prod(qz, x)
    xt = o.decode_prod(qz, idx, bits, n, g)
    xm = o.mse_reconstruct(qz, "prod", idx, n)
    true = np.sum(q * x, axis=1)
    return np.sum(q * xt, axis=1) - true, np.sum(q * xm, axis=1) - true


@pytest.mark.parametrize("rho", [0.0, 0.9])
def test_qjl_unbiased_with_negative_control(rho):
    # E_S <q, x_tilde> = <q, x> (blog.hotdry.top, QJL section).  1e5 pairs in
    # 2000 batches, a fresh S per batch; the SE comes from batch means.  m is
    # chosen different from d so that the constant sqrt(pi/2)/m is pinned.
    d, m, batches, per = 16, 24, 2000, 50
    qz = o.Quantizer(d, 3, seed=11)
    rng = np.random.default_rng(12)
    S_all = o.normals(99, o.TAG_QJL, batches * m * d).reshape(batches, m, d)
    tq_means, mse_means = [], []
    for b in range(batches):
        u = _unit(rng, per, d)
        x = u * rng.uniform(0.5, 2.0, (per, 1))
        q = rho * math.sqrt(d) * u + math.sqrt(1 - rho ** 2) * rng.standard_normal((per, d))
        e_tq, e_mse = _tq_error_batch(qz, x, q, S_all[b])
        tq_means.append(e_tq.mean())
        mse_means.append(e_mse.mean())
    tq_means, mse_means = np.array(tq_means), np.array(mse_means)
    z_tq = tq_means.mean() / (tq_means.std(ddof=1) / math.sqrt(batches))
    z_mse = mse_means.mean() / (mse_means.std(ddof=1) / math.sqrt(batches))
    assert abs(z_tq) < 3.0
    if rho > 0:
        assert z_mse < -20.0      # the MSE-only estimate is biased towards 0


def test_qjl_wrong_constant_is_biased():
    # negative control for the constant: using /d instead of /m (m != d)
    # must show a bias at rho = 0.9
    d, m, batches, per = 16, 24, 400, 50
    qz = o.Quantizer(d, 3, seed=11)
    rng = np.random.default_rng(13)
    S_all = o.normals(7, o.TAG_QJL, batches * m * d).reshape(batches, m, d)
    means = []
    for b in range(batches):
        u = _unit(rng, per, d)
        q = 0.9 * math.sqrt(d) * u + math.sqrt(1 - 0.81) * rng.standard_normal((per, d))
        qz.s, qz.m = S_all[b], m
        idx, bits, n, g = o.encode_prod(qz, u)
        sig = 2.0 * bits - 1
        xt = o.mse_reconstruct(qz, "prod", idx, n) + (g * math.sqrt(math.pi / 2) / d)[:, None] * (sig @ S_all[b])
        means.append(np.mean(np.sum(q * xt, 1) - np.sum(q * u, 1)))
    means = np.array(means)
    assert abs(means.mean() / (means.std(ddof=1) / math.sqrt(batches))) > 5


def test_qjl_variance_closed_form():
    # Var_S <q, x_tilde> = [(pi/2) gamma^2 ||q||^2 - <q, r>^2] / m for Gaussian S
    d = m = 16
    trials = 20000
    qz = o.Quantizer(d, 2, seed=3)
    rng = np.random.default_rng(21)
    x = rng.standard_normal((1, d))
    q = rng.standard_normal((1, d))
    S_all = o.normals(1234, o.TAG_QJL, trials * m * d).reshape(trials, m, d)
    _, c, t = qz.codebook("prod")
    idx, _, n, _ = o.encode_prod(qz, x)
    r = x - o.mse_reconstruct(qz, "prod", idx, n)
    gam = np.linalg.norm(r)
    est = np.empty(trials)
    for k in range(trials):
        qz.s = S_all[k]
        i2, bits, n2, g2 = o.encode_prod(qz, x)
        est[k] = (q @ o.decode_prod(qz, i2, bits, n2, g2).T)[0, 0]
    want = (math.pi / 2 * gam ** 2 * np.sum(q * q) - float((q @ r.T)[0, 0]) ** 2) / m
    assert abs(est.var() / want - 1) < 4 * math.sqrt(2 / trials) + 0.01
    assert abs(est.mean() - float((q @ x.T)[0, 0])) < 4 * math.sqrt(want / trials)


@pytest.mark.parametrize("d,bits,n", [(128, 3, 37), (200, 2, 5), (200, 4, 3), (20, 4, 70)])
def test_prod_layout_roundtrip(d, bits, n):
    rng = np.random.default_rng(7)
    bp = bits - 1
    idx = rng.integers(0, 2 ** bp, (n, d))
    sg = rng.integers(0, 2, (n, d)).astype(np.uint8)
    w = o.pack_prod(idx, sg, bp, d)
    G = (d + 31) // 32
    assert w.shape == (n, G, bits) and w.dtype == np.uint32
    i2, s2 = o.unpack_prod(w, bp, d)
    assert np.array_equal(i2, idx) and np.array_equal(s2, sg)
    # bit i of word (g, p) is bit p of coordinate 32g+i
    j = min(d - 1, 37)
    assert ((int(w[0, j // 32, 0]) >> (j % 32)) & 1) == (idx[0, j] & 1)
    assert ((int(w[0, j // 32, bp]) >> (j % 32)) & 1) == sg[0, j]


@pytest.mark.parametrize("n,bp,d", [(1, 3, 128), (33, 3, 128), (64, 4, 16), (70, 1, 8)])
def test_mse_layout_roundtrip(n, bp, d):
    rng = np.random.default_rng(8)
    idx = rng.integers(0, 2 ** bp, (n, d))
    w = o.pack_mse(idx, bp, d)
    assert w.shape == ((n + 31) // 32, bp, d)
    assert np.array_equal(o.unpack_mse(w, n, bp, d), idx)
    t = n - 1
    assert ((int(w[t // 32, bp - 1, 3 % d]) >> (t % 32)) & 1) == ((idx[t, 3 % d] >> (bp - 1)) & 1)


def test_record_size_matches_page_compression_ratios(golden):
    # 3 and 2 total bits at d = 128 with fp32 norm + gamma: 256 B of fp16 per
    # key over 56 / 40 B -> 4.57x / 6.4x, the page's turbo3 / turbo2 figures.
    pv = golden["pages"]["compression_vs_fp16"]["values"]
    for bits in (2, 3):
        assert abs(256 / o.record_bytes("prod", 128, bits) - pv[str(bits)]) < 0.05


@pytest.mark.parametrize("d,bits", [(16, 2), (128, 3), (200, 4), (48, 1)])
def test_mse_keys_scores_equal_inner_product_with_decode_and_pack_roundtrip(d, bits):
    """MSE-only keys: the logit from indices equals <q, decode_mse(code)>
    (two routes), and the token-major packing round-trips."""
    rng = np.random.default_rng(d + bits)
    qz = o.Quantizer(d, bits, 3)
    x = rng.standard_normal((50, d)) * rng.uniform(0.5, 4.0, (50, 1))
    q = rng.standard_normal((7, d))
    idx, nrm = o.encode_mse(qz, x)
    ref = q @ o.decode_mse(qz, idx, nrm).T
    np.testing.assert_allclose(o.scores_mse(qz, q, idx, nrm), ref, rtol=1e-10, atol=1e-10 * np.abs(ref).max())
    w = o.pack_mse_keys(idx, bits, d)
    assert w.shape == (50, (d + 31) // 32, bits)
    assert np.array_equal(o.unpack_mse_keys(w.reshape(50, -1), bits, d), idx)
    assert o.record_bytes("mse_keys", d, bits) == w[0].nbytes + 4
