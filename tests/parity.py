"""Comparison helpers for the GPU-vs-oracle parity tests.

Tolerances (the method's parity bar):
  codes   bit-exact (all layouts: prod keys, MSE-only keys, values), except
          an MSE index whose oracle rotated coordinate lies
          within 1e-5 of a decision threshold may take the adjacent index,
          and a QJL bit whose oracle projection |z| < 1e-5 * gamma may flip;
          at most 1e-4 of all coded coordinates may differ.  When an index
          differs, the oracle's QJL bits and gamma are recomputed from the
          GPU's indices before they are compared (cascade rule).
  norms, gammas   1e-5 relative.
  logits  |gpu - oracle| <= 1e-3 * max(|oracle|, ||q|| n / sqrt(d)), on
          identical codes (the GPU's codes fed to the oracle).
  attention output, per row: |gpu - oracle| <= 1e-3 * max(|oracle_e|, ||oracle_row|| / sqrt(d)).
  top-k   indices distinct and in range, scores non-increasing, each score
          within the logit tolerance of the oracle's logit at that index; the
          set equals the oracle's top k except for swaps among keys whose
          oracle scores lie within the logit tolerance of the oracle's k-th.
"""
import math

import numpy as np

from oracle import tq_oracle as o

BAND = 1e-5
MAX_FLIP_FRAC = 1e-4


def to_u32(t):
    return t.detach().cpu().numpy().view(np.uint32)


def _threshold_distance(qz, x, n_o, t, where):
    """Distance of the oracle's rotated coordinate y = Pi x / ||x|| to the
    nearest decision threshold, at the coordinates selected by `where`."""
    rows = np.any(where, axis=1) & (n_o > 0)
    y = np.zeros(x.shape)
    y[rows] = (x[rows] / n_o[rows, None]) @ qz.pi.T
    return np.min(np.abs(y[where][:, None] - t[None, :]), axis=-1)


def check_prod_codes(qz, x, codes, norms, gammas):
    """qz: oracle Quantizer; x float64 [N, d]; GPU outputs as numpy.  Returns
    (idx_gpu, bits_gpu, stats)."""
    d = qz.d
    bp, c, t = qz.codebook("prod")
    N = x.shape[0]
    idx_g, bits_g = o.unpack_prod(codes.reshape(N, -1), bp, d)
    idx_o, bits_o, n_o, g_o = o.encode_prod(qz, x)
    bad_idx = idx_g != idx_o
    assert np.all(np.abs(idx_g - idx_o)[bad_idx] == 1), "index differs by more than one level"
    dist = _threshold_distance(qz, x, n_o, t, bad_idx)
    assert np.all(dist < BAND), f"index flips outside the band: {np.sum(dist >= BAND)}"
    # cascade rule: recompute sketch and gamma from the GPU's indices where they differ
    rows = np.any(bad_idx, axis=1)
    bits_ref = bits_o.copy()
    g_ref = g_o.copy()
    _, _, z_all = o.qjl_from_indices(qz, x, idx_o)
    if rows.any():
        b2, g2, z2 = o.qjl_from_indices(qz, x[rows], idx_g[rows])
        bits_ref[rows] = b2
        g_ref[rows] = g2
        z_all[rows] = z2
    bad_bit = bits_g != bits_ref
    zb = np.abs(z_all) < BAND * g_ref[:, None]
    assert np.all(zb[bad_bit]), f"QJL bits flipped outside the band: {np.sum(~zb[bad_bit])}"
    flips = int(bad_idx.sum() + bad_bit.sum())
    assert flips <= MAX_FLIP_FRAC * N * (d + qz.m) + 0.5, f"{flips} flipped coordinates"
    assert np.allclose(norms, n_o, rtol=1e-5, atol=1e-30)
    pos = g_ref > 0
    assert np.all(gammas[~pos] == 0)
    if pos.any():
        assert np.max(np.abs(gammas[pos] - g_ref[pos]) / g_ref[pos]) < 1e-5
    return idx_g, bits_g, {"index_flips": int(bad_idx.sum()), "bit_flips": int(bad_bit.sum())}


def check_mse_codes(qz, x, codes, norms):
    d = qz.d
    bp, c, t = qz.codebook("mse")
    N = x.shape[0]
    idx_g = o.unpack_mse(codes, N, bp, d)
    idx_o, n_o = o.encode_mse(qz, x)
    bad = idx_g != idx_o
    assert np.all(np.abs(idx_g - idx_o)[bad] == 1)
    dist = _threshold_distance(qz, x, n_o, t, bad)
    assert np.all(dist < BAND), f"index flips outside the band: {np.sum(dist >= BAND)}"
    assert bad.sum() <= MAX_FLIP_FRAC * N * d + 0.5
    assert np.allclose(norms, n_o, rtol=1e-5, atol=1e-30)
    # padding tokens of the last block must be zero bits
    nb = (N + 31) // 32
    if N % 32:
        w = codes.reshape(nb, bp, d)[-1]
        assert np.all((w >> np.uint32(N % 32)) == 0)
    return idx_g, {"index_flips": int(bad.sum())}


def check_mse_key_codes(qz, x, codes, norms):
    """MSE-only keys (token major, all bits to the index): the mse-values
    rules (band, flip budget, norms); unused bits of the last group are 0."""
    d = qz.d
    bp, c, t = qz.codebook("mse")
    N = x.shape[0]
    G = (d + 31) // 32
    words = codes.reshape(N, G, bp)
    idx_g = o.unpack_mse_keys(words.reshape(N, -1), bp, d)
    idx_o, n_o = o.encode_mse(qz, x)
    bad = idx_g != idx_o
    assert np.all(np.abs(idx_g - idx_o)[bad] == 1)
    dist = _threshold_distance(qz, x, n_o, t, bad)
    assert np.all(dist < BAND), f"index flips outside the band: {np.sum(dist >= BAND)}"
    assert bad.sum() <= MAX_FLIP_FRAC * N * d + 0.5
    assert np.allclose(norms, n_o, rtol=1e-5, atol=1e-30)
    if d % 32:
        assert np.all((words[:, -1, :] >> np.uint32(d % 32)) == 0), "bits past d must be 0"
    return idx_g, {"index_flips": int(bad.sum())}


def check_logits(gpu, ref, qnorm, knorm, d, rel=1e-3):
    """gpu/ref [Q, N]; qnorm [Q]; knorm [N]."""
    floor = qnorm[:, None] * knorm[None, :] / math.sqrt(d)
    tol = rel * np.maximum(np.abs(ref), floor)
    err = np.abs(gpu - ref)
    worst = float(np.max(err / np.maximum(np.maximum(np.abs(ref), floor), 1e-30)))
    assert np.all(err <= tol + 1e-30), f"logit error {worst:.3g} (relative to the floor) exceeds {rel}"
    return worst


def check_attention(gpu, ref, rel=1e-3):
    """gpu/ref [R, d]."""
    d = ref.shape[1]
    floor = np.linalg.norm(ref, axis=1, keepdims=True) / math.sqrt(d)
    tol = rel * np.maximum(np.abs(ref), floor)
    err = np.abs(gpu - ref)
    worst = float(np.max(err / np.maximum(np.maximum(np.abs(ref), floor), 1e-30)))
    assert np.all(err <= tol + 1e-30), f"attention error {worst:.3g} exceeds {rel}"
    return worst


def check_topk(gpu_s, gpu_i, ref, qnorm, knorm, d, rel=1e-3):
    """gpu_s/gpu_i [Q, k] (GPU top-k); ref [Q, N] oracle logits on identical
    codes; qnorm [Q]; knorm [N].  Returns the number of allowed swaps."""
    Q, k = gpu_i.shape
    N = ref.shape[1]
    swaps = 0
    ref_s, ref_i = o.topk(ref, k)
    for r in range(Q):
        gi = gpu_i[r].astype(np.int64)
        assert np.all((gi >= 0) & (gi < N)), "top-k index out of range"
        assert len(set(gi.tolist())) == k, "top-k indices repeat"
        assert np.all(np.diff(gpu_s[r]) <= 0), "top-k scores not in descending order"
        tol_all = rel * np.maximum(np.abs(ref[r]), qnorm[r] * knorm / math.sqrt(d))
        err = np.abs(gpu_s[r] - ref[r, gi])
        assert np.all(err <= tol_all[gi] + 1e-30), f"query {r}: top-k score off its oracle logit"
        kth = ref_i[r, -1]
        gset, rset = set(gi.tolist()), set(ref_i[r].tolist())
        for i in gset - rset:      # chosen by the GPU, not by the oracle
            assert ref[r, i] >= ref[r, kth] - tol_all[i] - tol_all[kth], f"query {r}: key {i} is not a top-{k} key"
        for i in rset - gset:      # chosen by the oracle, missed by the GPU
            assert ref[r, i] <= ref[r, kth] + tol_all[i] + tol_all[kth], f"query {r}: top-{k} key {i} missed"
        swaps += len(gset - rset)
    return swaps
