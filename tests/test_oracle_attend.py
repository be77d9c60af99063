"""Pins for the oracle's decode attention and top-k (CPU only).

Attention over the packed cache is the textbook scaled-dot-product softmax
over logits from codes (keys) and MSE-decoded values, with the most recent
tokens optionally kept exact (blog.hotdry.top, engineering configuration:
keep the latest 128-256 tokens in full precision).
"""
import math

import numpy as np
import pytest
from scipy import special

from oracle import tq_oracle as o


def _setup(N=96, T=8, d=32, G=4, seed=0):
    rng = np.random.default_rng(seed)
    kq = o.Quantizer(d, 3, seed=1)
    vq = o.Quantizer(d, 3, seed=2)
    K = rng.standard_normal((N, d)) * 3
    V = rng.standard_normal((N, d))
    q = rng.standard_normal((G, d))
    ki, kb, kn, kg = o.encode_prod(kq, K)
    vi, vn = o.encode_mse(vq, V)
    kt = rng.standard_normal((T, d))
    vt = rng.standard_normal((T, d))
    return kq, vq, q, (ki, kb, kn, kg), (vi, vn), kt, vt


def test_attend_equals_dense_textbook_attention():
    kq, vq, q, (ki, kb, kn, kg), (vi, vn), kt, vt = _setup()
    out = o.attend(kq, vq, q, ki, kb, kn, kg, vi, vn, kt, vt)
    # dense: decoded keys and values as matrices, scipy softmax
    Kd = np.concatenate([o.decode_prod(kq, ki, kb, kn, kg), kt])
    Vd = np.concatenate([o.decode_mse(vq, vi, vn), vt])
    p = special.softmax(q @ Kd.T / math.sqrt(q.shape[1]), axis=1)
    assert np.max(np.abs(out - p @ Vd)) < 1e-12


def test_attend_without_tail_and_custom_scale():
    kq, vq, q, (ki, kb, kn, kg), (vi, vn), _, _ = _setup(seed=1)
    out = o.attend(kq, vq, q, ki, kb, kn, kg, vi, vn, scale=0.05)
    Kd = o.decode_prod(kq, ki, kb, kn, kg)
    Vd = o.decode_mse(vq, vi, vn)
    p = special.softmax(0.05 * q @ Kd.T, axis=1)
    assert np.max(np.abs(out - p @ Vd)) < 1e-12


def test_attend_zero_scale_is_mean():
    kq, vq, q, (ki, kb, kn, kg), (vi, vn), kt, vt = _setup(seed=2)
    out = o.attend(kq, vq, q, ki, kb, kn, kg, vi, vn, kt, vt, scale=0.0)
    Vd = np.concatenate([o.decode_mse(vq, vi, vn), vt])
    assert np.max(np.abs(out - Vd.mean(0)[None])) < 1e-12


def test_attend_dominant_logit_picks_its_value():
    kq, vq, q, (ki, kb, kn, kg), (vi, vn), kt, vt = _setup(seed=3)
    kt2 = kt.copy()
    kt2[5] = q[0] * 1e3          # one tail key aligned with query 0, huge logit
    out = o.attend(kq, vq, q[:1], ki, kb, kn, kg, vi, vn, kt2, vt)
    assert np.max(np.abs(out[0] - vt[5])) < 1e-9


def test_attend_softmax_is_shift_invariant_and_rows_sum_to_one():
    kq, vq, q, (ki, kb, kn, kg), (vi, vn), kt, vt = _setup(seed=4)
    ones = np.ones_like(vt)
    vones_i, vones_n = o.encode_mse(vq, np.ones((len(vi), q.shape[1])))
    out = o.attend(kq, vq, q, ki, kb, kn, kg, vones_i, vones_n, kt, ones)
    # values all equal to the MSE decode of the all-ones vector / ones
    dec = o.decode_mse(vq, vones_i, vones_n)[0]
    assert np.all(out.min(0) >= np.minimum(dec, 1).min() - 1e-12)


def test_topk_matches_full_sort_and_tie_order():
    rng = np.random.default_rng(5)
    lg = rng.standard_normal((7, 500))
    lg[3, 10] = lg[3, 20] = lg[3].max() + 1.0          # a tie at the top
    s, i = o.topk(lg, 10)
    for r in range(7):
        order = sorted(range(500), key=lambda j: (-lg[r, j], j))[:10]
        assert list(i[r]) == order
        assert np.array_equal(s[r], lg[r, order])
    assert list(i[3, :2]) == [10, 20]


def test_scores_gqa_head_mapping():
    rng = np.random.default_rng(6)
    qz = o.Quantizer(16, 3, seed=0)
    B, Hkv, G, N, d = 2, 3, 2, 40, 16
    X = rng.standard_normal((B, Hkv, N, d))
    q = rng.standard_normal((B, Hkv * G, d))
    enc = [[o.encode_prod(qz, X[b, h]) for h in range(Hkv)] for b in range(B)]
    idx = np.array([[e[0] for e in r] for r in enc])
    bits = np.array([[e[1] for e in r] for r in enc])
    nrm = np.array([[e[2] for e in r] for r in enc])
    gam = np.array([[e[3] for e in r] for r in enc])
    out = o.scores_gqa(qz, q, idx, bits, nrm, gam)
    for b in range(B):
        for h in range(Hkv * G):
            kv = h // G
            ref = q[b, h] @ o.decode_prod(qz, idx[b, kv], bits[b, kv], nrm[b, kv], gam[b, kv]).T
            assert np.max(np.abs(out[b, h] - ref)) < 1e-10 * np.abs(ref).max()


def test_topk_parity_helper_accepts_ties_and_rejects_wrong_keys():
    """The top-k comparison used by the GPU tests: the oracle's own answer
    passes, a swap inside the tolerance passes, a clearly worse key fails."""
    from tests import parity as P
    rng = np.random.default_rng(3)
    ref = rng.standard_normal((2, 500))
    ref[0, 7] = ref[0, 9] = 5.0            # a tie at the boundary of the top 2 ...
    ref[0, 3] = 6.0
    s, i = o.topk(ref, 2)
    qn, kn = np.ones(2), np.ones(500)
    assert P.check_topk(s.astype(np.float32), i, ref, qn, kn, 16) == 0
    i2 = i.copy()
    i2[0, 1] = 9                           # ... may resolve either way
    assert P.check_topk(ref[np.arange(2)[:, None], i2].astype(np.float32), i2, ref, qn, kn, 16) == 1
    i3 = i.copy()
    i3[1, 1] = int(np.argmin(ref[1]))      # the worst key is no top-2 key
    with pytest.raises(AssertionError):
        P.check_topk(ref[np.arange(2)[:, None], i3].astype(np.float32), i3, ref, qn, kn, 16)


def _sparse_case(seed, tau, spread=3.0):
    kq, vq, q, (ki, kb, kn, kg), (vi, vn), kt, vt = _setup(N=300, seed=seed)
    q = q * spread
    return kq, vq, q, (ki, kb, kn, kg), (vi, vn), kt, vt


def test_sparse_v_threshold_zero_drops_nothing():
    kq, vq, q, (ki, kb, kn, kg), (vi, vn), kt, vt = _sparse_case(5, 0.0)
    p, D = o.sparse_v_dropset(kq, vq, q, ki, kb, kn, kg, vi, vn, 0.0, kt, vt)
    assert not D.any()
    assert np.allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert np.max(o.sparse_v_bound(kq, vq, q, ki, kb, kn, kg, vi, vn, 0.0, kt, vt)) == 0.0


@pytest.mark.parametrize("tau", [1e-4, 1e-2, 0.3])
def test_sparse_v_bound_covers_every_allowed_drop(tau):
    # Any subset S of the drop set D, removed from the value sum of the dense
    # textbook attention (decoded matrices, scipy softmax, values of S set to
    # 0), moves each output element by at most the oracle's bound.
    kq, vq, q, (ki, kb, kn, kg), (vi, vn), kt, vt = _sparse_case(6, tau)
    d = q.shape[1]
    Kd = np.concatenate([o.decode_prod(kq, ki, kb, kn, kg), kt])
    Vd = np.concatenate([o.decode_mse(vq, vi, vn), vt])
    p = special.softmax(q @ Kd.T / math.sqrt(d), axis=1)
    dense = p @ Vd
    _, D = o.sparse_v_dropset(kq, vq, q, ki, kb, kn, kg, vi, vn, tau, kt, vt)
    bound = o.sparse_v_bound(kq, vq, q, ki, kb, kn, kg, vi, vn, tau, kt, vt)
    assert D.any()
    rng = np.random.default_rng(7)
    for trial in range(6):
        for r in range(len(q)):
            S = D[r] & (rng.random(D.shape[1]) < (1.0 if trial == 0 else 0.5))
            V2 = Vd.copy()
            V2[:len(vi)][S] = 0.0
            out = p[r] @ V2
            assert np.all(np.abs(out - dense[r]) <= bound[r] + 1e-12)
    # the whole of D reaches the bound on some element only when the dropped
    # terms share a sign there; it is never exceeded
    assert np.all(bound >= 0)


def test_sparse_v_running_max_drops_a_subset():
    # The rule against the running maximum of the chunk (sequence order,
    # 16-token steps, each step's maximum included before its tokens are
    # judged) never drops a token outside D: the running maximum is at most
    # the overall one.  Written here as a plain loop, independent of the
    # oracle's set construction.
    tau = 0.05
    kq, vq, q, (ki, kb, kn, kg), (vi, vn), kt, vt = _sparse_case(8, tau, spread=5.0)
    d = q.shape[1]
    logit = o.scores(kq, q, ki, kb, kn, kg)
    _, D = o.sparse_v_dropset(kq, vq, q, ki, kb, kn, kg, vi, vn, tau, None, None)
    for r in range(len(q)):
        s = logit[r] / math.sqrt(d)
        w = np.exp(s - s.max()) * vn
        run = 0.0
        for t0 in range(0, len(s), 16):
            run = max(run, w[t0:t0 + 16].max())
            drop = w[t0:t0 + 16] < tau * run
            assert np.all(D[r, t0:t0 + 16][drop])


def test_sparse_v_dropset_grows_with_the_threshold():
    kq, vq, q, (ki, kb, kn, kg), (vi, vn), kt, vt = _sparse_case(9, 0.0)
    sets = [o.sparse_v_dropset(kq, vq, q, ki, kb, kn, kg, vi, vn, tau, kt, vt)[1] for tau in (1e-6, 1e-3, 0.1, 0.9)]
    for a, b in zip(sets, sets[1:]):
        assert np.all(b[a])
