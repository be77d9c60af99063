"""Pins for the oracle's residual sketch recomputed from given indices
(qjl_from_indices), which the parity rule uses whenever a GPU index sits on
the other side of a decision threshold (CPU only).

The residual of a key is r = x - x_hat with x_hat = n Pi^T c[idx] and its
sketch is sign(S r), gamma = ||r|| (blog.hotdry.top, "TurboQuant
vector-search compression", QJL residual correction section).  The checks
below do not go through the oracle's reconstruction:

  * rotated frame: Pi is orthogonal, so r = n Pi^T (y - c[idx]) with
    y = Pi x / n, gamma = n ||y - c[idx]|| and S r = n (S Pi^T)(y - c[idx]);
  * one index moved by one level: x_hat moves by n (c[a'] - c[a]) times row j
    of Pi, so the new residual is the old one minus that vector;
  * d = 3, written out with explicit loops;
  * special cases: the encoder's own indices reproduce its sketch, and the
    zero vector gives gamma = 0 with every bit 1 (sign(0) = +1).
"""
import numpy as np
import pytest

from oracle import tq_oracle as o


def _keys(d, n, seed):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((n, d)) * rng.uniform(0.5, 20.0, (n, 1))


@pytest.mark.parametrize("d,bits", [(16, 2), (128, 3), (200, 4)])
def test_own_indices_reproduce_the_encoder(d, bits):
    qz = o.Quantizer(d, bits, 3)
    x = _keys(d, 300, d + bits)
    idx, b01, _, gam = o.encode_prod(qz, x)
    b2, g2, z2 = o.qjl_from_indices(qz, x, idx)
    assert np.array_equal(b2, b01)
    assert np.array_equal(g2, gam)
    assert np.array_equal(b2, (z2 >= 0).astype(np.uint8))


@pytest.mark.parametrize("d,bits", [(16, 2), (128, 3), (64, 4)])
def test_rotated_frame_identity(d, bits):
    """gamma = n ||y - c[idx]|| and z = n S Pi^T (y - c[idx]) for arbitrary
    (not nearest) indices."""
    qz = o.Quantizer(d, bits, 5)
    _, c, _ = qz.codebook("prod")
    rng = np.random.default_rng(d)
    x = _keys(d, 200, d * 3)
    idx = rng.integers(0, len(c), size=x.shape)
    n = np.linalg.norm(x, axis=1)
    y = (x / n[:, None]) @ qz.pi.T
    rho = y - c[idx]
    _, g2, z2 = o.qjl_from_indices(qz, x, idx)
    np.testing.assert_allclose(g2, n * np.linalg.norm(rho, axis=1), rtol=1e-12)
    sp = qz.s @ qz.pi.T
    np.testing.assert_allclose(z2, n[:, None] * (rho @ sp.T), rtol=1e-9, atol=1e-9 * n.max())


@pytest.mark.parametrize("up", [True, False])
def test_one_index_moved_by_a_level(up):
    d, bits = 128, 3
    qz = o.Quantizer(d, bits, 0)
    _, c, _ = qz.codebook("prod")
    x = _keys(d, 50, 11)
    idx, _, n, _ = o.encode_prod(qz, x)
    _, g0, z0 = o.qjl_from_indices(qz, x, idx)
    r0 = x - n[:, None] * (c[idx] @ qz.pi)
    rng = np.random.default_rng(1)
    for i in range(len(x)):
        j = int(rng.integers(d))
        a = int(idx[i, j])
        a2 = a + 1 if (up and a + 1 < len(c)) or a == 0 else a - 1
        moved = idx[i:i + 1].copy()
        moved[0, j] = a2
        b2, g2, z2 = o.qjl_from_indices(qz, x[i:i + 1], moved)
        r_hand = r0[i] - n[i] * (c[a2] - c[a]) * qz.pi[j]
        assert abs(g2[0] - np.linalg.norm(r_hand)) <= 1e-12 * np.linalg.norm(x[i])
        np.testing.assert_allclose(z2[0], qz.s @ r_hand, rtol=1e-10, atol=1e-10 * np.abs(z0[i]).max())
        assert np.array_equal(b2[0], (qz.s @ r_hand >= 0).astype(np.uint8))
        # the moved index makes the residual longer (the encoder's index is the nearest)
        assert g2[0] >= g0[i] - 1e-12 * np.linalg.norm(x[i])


def test_d3_written_out():
    d, bits = 3, 2
    qz = o.Quantizer(d, bits, 9)
    _, c, _ = qz.codebook("prod")
    x = np.array([[1.0, -2.0, 0.5], [0.1, 0.2, -0.3], [4.0, 0.0, 0.0]])
    idx = np.array([[0, 1, 1], [1, 0, 1], [1, 1, 0]])
    b2, g2, z2 = o.qjl_from_indices(qz, x, idx)
    for i in range(3):
        n = (x[i, 0] ** 2 + x[i, 1] ** 2 + x[i, 2] ** 2) ** 0.5
        xh = [0.0, 0.0, 0.0]
        for k in range(3):            # x_hat_k = n sum_j Pi[j][k] c[idx_j]
            for j in range(3):
                xh[k] += n * qz.pi[j][k] * c[idx[i][j]]
        r = [x[i][k] - xh[k] for k in range(3)]
        assert abs(g2[i] - (r[0] ** 2 + r[1] ** 2 + r[2] ** 2) ** 0.5) < 1e-12
        for row in range(3):
            z = qz.s[row][0] * r[0] + qz.s[row][1] * r[1] + qz.s[row][2] * r[2]
            assert abs(z2[i, row] - z) < 1e-12
            assert b2[i, row] == (1 if z >= 0 else 0)


def test_zero_vector():
    qz = o.Quantizer(32, 3, 0)
    _, c, _ = qz.codebook("prod")
    x = np.zeros((1, 32))
    idx = np.full((1, 32), len(c) // 2 - 1)
    b2, g2, _ = o.qjl_from_indices(qz, x, idx)
    assert g2[0] == 0.0 and np.all(b2 == 1)
