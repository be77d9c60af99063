"""Pins for the oracle's segmented cache (temporal decay), re-quantization
and fractional widths (CPU only).

Temporal decay (ai-coding.wiselychen.com, TurboQuant+ section: older tokens
kept at a lower precision) is read as a cache in age segments, each with its
own quantizers, sharing one softmax; a token ages by being decoded at its old
width and encoded again at the new one.  Fractional widths (blog.hotdry.top,
engineering configuration: 3.5-bit = 3-bit MSE + 1-bit QJL) are read as the
mean width over the cached keys and values.
"""
import math

import numpy as np
import pytest
from scipy import special

from oracle import tq_oracle as o


def _segment(kq, vq, x_k, x_v, mse_keys=False):
    if mse_keys:
        ki, kn = o.encode_mse(kq, x_k)
        kb, kg = None, None
    else:
        ki, kb, kn, kg = o.encode_prod(kq, x_k)
    vi, vn = o.encode_mse(vq, x_v)
    return (kq, vq, ki, kb, kn, kg, vi, vn)


def _data(d, n, seed):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((n, d)) * 3.0, rng.standard_normal((n, d)), rng.standard_normal((4, d)) * 0.3


def test_one_segment_is_attend():
    d = 32
    kq, vq = o.Quantizer(d, 3, 0), o.Quantizer(d, 3, 1)
    xk, xv, q = _data(d, 300, 1)
    seg = _segment(kq, vq, xk, xv)
    tk, tv = xk[:7] * 0.5, xv[:7]
    a = o.attend_segments([seg], q, tk, tv)
    b = o.attend(kq, vq, q, seg[2], seg[3], seg[4], seg[5], seg[6], seg[7], tk, tv)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)


def test_segment_order_and_split_invariance():
    d = 32
    k4, v4 = o.Quantizer(d, 4, 0), o.Quantizer(d, 4, 1)
    k2, v2 = o.Quantizer(d, 2, 0), o.Quantizer(d, 2, 1)
    xk, xv, q = _data(d, 500, 2)
    old = _segment(k2, v2, xk[:300], xv[:300])
    new = _segment(k4, v4, xk[300:], xv[300:])
    a = o.attend_segments([old, new], q)
    b = o.attend_segments([new, old], q)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)
    # the old segment cut in two pieces (same quantizers) changes nothing
    o1 = (k2, v2) + tuple(t[:120] for t in old[2:])
    o2 = (k2, v2) + tuple(t[120:] for t in old[2:])
    c = o.attend_segments([o1, new, o2], q)
    np.testing.assert_allclose(a, c, rtol=1e-12, atol=1e-14)


def test_segments_against_textbook_attention_on_decoded_tensors():
    """softmax(scale q K~^T) V^ with K~ the decoded keys (each segment by its
    own quantizer, <q, decode(k)> being the logit) and V^ the decoded values,
    with scipy's softmax; MSE-only keys in one segment."""
    d = 16
    xk, xv, q = _data(d, 400, 3)
    segs = [_segment(o.Quantizer(d, 4, 0), o.Quantizer(d, 3, 1), xk[:100], xv[:100]),
            _segment(o.Quantizer(d, 2, 5), o.Quantizer(d, 2, 6), xk[100:300], xv[100:300]),
            _segment(o.Quantizer(d, 3, 7), o.Quantizer(d, 1, 8), xk[300:], xv[300:], mse_keys=True)]
    tk, tv = xk[:5], xv[:5]
    K, V = [], []
    for (kq, vq, ki, kb, kn, kg, vi, vn) in segs:
        K.append(o.decode_mse(kq, ki, kn) if kb is None else o.decode_prod(kq, ki, kb, kn, kg))
        V.append(o.decode_mse(vq, vi, vn))
    K = np.concatenate(K + [tk])
    V = np.concatenate(V + [tv])
    ref = special.softmax((q @ K.T) / math.sqrt(d), axis=1) @ V
    np.testing.assert_allclose(o.attend_segments(segs, q, tk, tv), ref, rtol=1e-10, atol=1e-12)
    # scale -> 0: the uniform mean of every value of every segment
    np.testing.assert_allclose(o.attend_segments(segs, q, tk, tv, scale=1e-300),
                               np.broadcast_to(V.mean(axis=0), ref.shape), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("d,b_from,b_to", [(64, 4, 2), (128, 3, 2), (32, 2, 1)])
def test_requantize_values_rotated_frame_closed_form(d, b_from, b_to):
    """Values whose quantizers share Pi (same d and seed): the decoded vector is
    n Pi^T c[idx], so its norm is n ||c[idx]|| and its rotated unit vector is
    c[idx] / ||c[idx]|| -- the new index is that bucketized by the new
    codebook, with no rotation at all."""
    qf, qt = o.Quantizer(d, b_from, 4), o.Quantizer(d, b_to, 4)
    _, cf, _ = qf.codebook("mse")
    _, _, tt = qt.codebook("mse")
    x = np.random.default_rng(d).standard_normal((200, d)) * 2.0
    idx, n = o.encode_mse(qf, x)
    idx2, n2 = o.requantize(qf, qt, "mse", idx, None, n, None)
    cn = np.linalg.norm(cf[idx], axis=1)
    np.testing.assert_allclose(n2, n * cn, rtol=1e-12)
    y = cf[idx] / cn[:, None]
    want = np.sum(y[..., None] > tt, axis=-1)
    dist = np.min(np.abs(y[..., None] - tt), axis=-1)
    assert np.all((idx2 == want) | (dist < 1e-12))


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_requantize_to_the_same_quantizer_keeps_the_indices(bits):
    """c[idx] / ||c[idx]|| lies in the cell of c[idx] (||c[idx]|| is sqrt(1 - D)
    up to fluctuation, so every centroid moves outward by a few percent, far
    less than the distance to its cell's edge): the indices are a fixed
    point."""
    d = 128
    qz = o.Quantizer(d, bits, 2)
    x = np.random.default_rng(bits).standard_normal((300, d))
    idx, n = o.encode_mse(qz, x)
    idx2, n2 = o.requantize(qz, qz, "mse", idx, None, n, None)
    assert np.array_equal(idx2, idx)


def test_requantized_keys_stay_unbiased():
    """A prod key aged from 4 to 2 bits: over fresh quantizer seeds of the new
    width the new logit is an unbiased estimate of <q, x~>, the old key's
    decoded value (the QJL estimator of the new quantizer applied to x~)."""
    d = 32
    rng = np.random.default_rng(9)
    x = rng.standard_normal((1, d))
    q = x * 0.8 + 0.6 * rng.standard_normal((1, d))
    q_old = o.Quantizer(d, 4, 100)
    idx, b01, n, g = o.encode_prod(q_old, x)
    x_old = o.decode_prod(q_old, idx, b01, n, g)
    target = float((q @ x_old.T)[0, 0])
    errs = []
    for s in range(3000):
        qn = o.Quantizer(d, 2, 1000 + s)
        i2, b2, n2, g2 = o.requantize(q_old, qn, "prod", idx, b01, n, g)
        errs.append(float(o.scores(qn, q, i2, b2, n2, g2)[0, 0]) - target)
    errs = np.array(errs)
    assert abs(errs.mean()) <= 3 * errs.std() / math.sqrt(len(errs))


def test_fractional_widths_follow_the_page_decomposition(golden):
    fw = golden["pages"]["fractional_widths"]["values"]
    kb, vb = o.kv_width_config(3.5)
    assert kb - 1 == fw["3.5"]["mse_bits"] and (kb + vb) / 2 == 3.5
    assert o.kv_width_config(2.5) == (3, 2)
    for w in (1.5, 2.0, 2.5, 3.0, 3.5, 4.0):
        kb, vb = o.kv_width_config(w)
        # mean stored bits per cached coordinate (key index + QJL bit, value index)
        assert ((kb - 1) + 1 + vb) / 2 == w
    with pytest.raises(ValueError):
        o.kv_width_config(2.75)


def test_decay_saving_in_the_page_range(golden):
    """Reading R28 with its benchmark setting -- the older two thirds of a
    long cache moved from 4-bit to 2-bit keys and values -- saves a share of
    the packed bytes inside the pages' 30-34%."""
    lo, hi = golden["pages"]["temporal_decay_saving"]["range"]
    d = 128
    rec = {b: o.record_bytes("prod", d, b) + o.record_bytes("mse", d, b) for b in (2, 4)}
    saving = (2 / 3) * (1 - rec[2] / rec[4])
    assert lo <= saving <= hi, saving
