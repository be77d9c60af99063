"""GPU parity: temporal decay (a cache kept in age segments at different
widths, one softmax) and re-quantization, through the C ABI, against the
oracle (attend_segments, requantize) on the same codes.

Tolerances as everywhere: attention per row |gpu - oracle| <= 1e-3
max(|oracle_e|, ||oracle_row||/sqrt(d)) on identical codes; re-quantized codes
bit-exact up to the decision band, judged against the oracle's encoding of the
oracle's float64 decode of the GPU's input codes.
"""
import numpy as np
import pytest

from oracle import tq_oracle as o
from tests import parity as P
from vector_quantization_tq_amd import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from vector_quantization_tq_amd import tq  # noqa: E402

_QZ = {}


def _pair(d, bits, seed, key_mode=tq.TQ_PROD):
    key = (d, bits, seed, key_mode)
    if key not in _QZ:
        g = tq.Quantizer(d, bits, seed)
        if key_mode != tq.TQ_PROD:
            g.set_key_mode(key_mode)
        _QZ[key] = (g, o.Quantizer(d, bits, seed))
    return _QZ[key]


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def _bf16(u16):
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).to(_dev()).view(torch.bfloat16)


def _make_segments(k, v, bounds, specs):
    """k, v: bf16 [nseq, N, d]; bounds: token ranges; specs: (key bits, key
    mode, value bits) per segment.  Value quantizers share seed 1 (one Pi);
    key quantizers seed 0."""
    segs, host = [], []
    d = k.shape[-1]
    for (a, b), (kb, km, vb) in zip(bounds, specs):
        gk, ok = _pair(d, kb, 0, km)
        gv, ov = _pair(d, vb, 1)
        kc, kn, kg = tq.tq_encode(gk, km, k[:, a:b].contiguous())
        vc, vn, _ = tq.tq_encode(gv, tq.TQ_MSE, v[:, a:b].contiguous())
        segs.append(tq.Segment(gk, gv, kc, kn, kg, vc, vn, b - a))
        n = b - a
        host.append((ok, ov, km, kb, vb, P.to_u32(kc), kn.cpu().numpy().astype(np.float64),
                     None if kg is None else kg.cpu().numpy().astype(np.float64), P.to_u32(vc),
                     vn.cpu().numpy().astype(np.float64), n,
                     gk.code_words(km, 1, n) if n else 0, gv.code_words(tq.TQ_MSE, 1, n) if n else 0, d))
    return segs, host


def _oracle_segments(host, s):
    out = []
    for (ok, ov, km, kb, vb, kw, kn, kg, vw, vn, n, per, perv, d) in host:
        if n == 0:
            continue
        sl = slice(s * n, (s + 1) * n)
        if km == tq.TQ_PROD:
            ki, kbits = o.unpack_prod(kw[s * per:(s + 1) * per].reshape(n, -1), kb - 1, d)
            kgs = kg[sl]
        else:
            ki, kbits, kgs = o.unpack_mse_keys(kw[s * per:(s + 1) * per].reshape(n, -1), kb, d), None, None
        vi = o.unpack_mse(vw[s * perv:(s + 1) * perv], n, vb, d)
        out.append((ok, ov, ki, kbits, kn[sl], kgs, vi, vn[sl]))
    return out


def _check_all(out, host, q, kf, vf, B, Hkv, Hq, n_tail, groups=None):
    G = Hq // Hkv
    N = kf.shape[1]
    worst = 0.0
    for (b, h) in (groups or [(b, h) for b in range(B) for h in range(Hkv)]):
        s = b * Hkv + h
        tails = (kf[s, N - n_tail:], vf[s, N - n_tail:]) if n_tail else (None, None)
        ref = o.attend_segments(_oracle_segments(host, s), q[b, h * G:(h + 1) * G], *tails)
        worst = max(worst, P.check_attention(out[b, h * G:(h + 1) * G], ref))
    return worst


def test_one_segment_is_attend_decode():
    print("case: segments one segment == tq_attend_decode", flush=True)
    B, Hkv, Hq, N = 2, 4, 16, 3000
    a = W._gqa_tensors(np.random.default_rng(5), B, Hkv, Hq, N, 128)
    k, v, q = _bf16(a["k_bf16"]).view(B * Hkv, N, 128), _bf16(a["v_bf16"]).view(B * Hkv, N, 128), _bf16(a["q_bf16"])
    segs, _ = _make_segments(k, v, [(0, N - 100)], [(3, tq.TQ_PROD, 3)])
    kt = k[:, N - 100:].contiguous().view(B, Hkv, 100, 128)
    vt = v[:, N - 100:].contiguous().view(B, Hkv, 100, 128)
    g = segs[0]
    ref = tq.tq_attend_decode(g.kq, g.vq, q, g.kcodes, g.knorms, g.kgammas, g.vcodes, g.vnorms, Hkv, g.n, kt, vt)
    out = tq.tq_attend_decode_segments(segs, q, Hkv, kt, vt)
    torch.cuda.synchronize()
    assert torch.equal(ref, out)


@pytest.mark.parametrize("B,Hkv,Hq,N,tail,bounds,specs", [
    (2, 4, 16, 4000, 64, [(0, 2936), (2936, 3936)], [(2, tq.TQ_PROD, 2), (4, tq.TQ_PROD, 4)]),
    (1, 2, 8, 5000, 0, [(0, 1000), (1000, 1001), (1001, 3000), (3000, 5000)],
     [(2, tq.TQ_PROD, 1), (3, tq.TQ_PROD, 2), (3, tq.TQ_MSE_KEYS, 3), (4, tq.TQ_PROD, 4)]),
    (1, 8, 32, 2000, 17, [(0, 0), (0, 1983)], [(4, tq.TQ_PROD, 4), (3, tq.TQ_PROD, 2)]),
])
def test_segments_against_oracle(B, Hkv, Hq, N, tail, bounds, specs):
    """Two to four segments at different key and value widths (one with
    MSE-only keys, one of a single token, one empty) and a bf16 tail; every
    group checked."""
    print(f"case: segments B={B} Hkv={Hkv} Hq={Hq} N={N} tail={tail} specs={specs}", flush=True)
    a = W._gqa_tensors(np.random.default_rng(N + tail), B, Hkv, Hq, N, 128)
    k, v, q = _bf16(a["k_bf16"]).view(B * Hkv, N, 128), _bf16(a["v_bf16"]).view(B * Hkv, N, 128), _bf16(a["q_bf16"])
    segs, host = _make_segments(k, v, bounds, specs)
    kt = k[:, N - tail:].contiguous().view(B, Hkv, tail, 128) if tail else None
    vt = v[:, N - tail:].contiguous().view(B, Hkv, tail, 128) if tail else None
    out = tq.tq_attend_decode_segments(segs, q, Hkv, kt, vt).cpu().numpy()
    w = _check_all(out, host, a["q"].astype(np.float64), a["k"].reshape(B * Hkv, N, 128).astype(np.float64),
                   a["v"].reshape(B * Hkv, N, 128).astype(np.float64), B, Hkv, Hq, tail)
    print("worst relative error", w)


@pytest.mark.parametrize("d", [64, 96, 256])
def test_segments_other_head_dims(d):
    """Two segments (2-bit and 4-bit) and a bf16 tail at head dimensions other
    than 128: each segment's chunk-kernel launch and the merge at d."""
    print(f"case: segments d={d} B=1 Hkv=4 Hq=16 N=6000 tail=40", flush=True)
    B, Hkv, Hq, N, tail = 1, 4, 16, 6000, 40
    a = W._gqa_tensors(np.random.default_rng(d), B, Hkv, Hq, N, d)
    k, v, q = _bf16(a["k_bf16"]).view(B * Hkv, N, d), _bf16(a["v_bf16"]).view(B * Hkv, N, d), _bf16(a["q_bf16"])
    segs, host = _make_segments(k, v, [(0, 3960), (3960, N - tail)], [(2, tq.TQ_PROD, 2), (4, tq.TQ_PROD, 4)])
    kt = k[:, N - tail:].contiguous().view(B, Hkv, tail, d)
    vt = v[:, N - tail:].contiguous().view(B, Hkv, tail, d)
    out = tq.tq_attend_decode_segments(segs, q, Hkv, kt, vt).cpu().numpy()
    w = _check_all(out, host, a["q"].astype(np.float64), a["k"].reshape(B * Hkv, N, d).astype(np.float64),
                   a["v"].reshape(B * Hkv, N, d).astype(np.float64), B, Hkv, Hq, tail)
    print("worst relative error", w)


def test_segments_full_size_long_context_decay():
    """The long-context layer (8 KV heads, 131072 tokens, last 256 bf16) with
    the older two thirds of the compressed tokens (87168) at 2-bit keys and
    values and the rest at 4 bits, as the benchmark runs it; every group
    checked."""
    print("case: segments long context decay 87168 @ 2-bit + 43648 @ 4-bit + 256 bf16", flush=True)
    wl = W.long_context()
    B, Hkv, Hq, N, tail = 1, 8, 32, 131072, 256
    k, v, q = (_bf16(wl.arrays["k_bf16"]).view(B * Hkv, N, 128), _bf16(wl.arrays["v_bf16"]).view(B * Hkv, N, 128),
               _bf16(wl.arrays["q_bf16"]))
    segs, host = _make_segments(k, v, [(0, 87168), (87168, N - tail)], [(2, tq.TQ_PROD, 2), (4, tq.TQ_PROD, 4)])
    kt = k[:, N - tail:].contiguous().view(B, Hkv, tail, 128)
    vt = v[:, N - tail:].contiguous().view(B, Hkv, tail, 128)
    out = tq.tq_attend_decode_segments(segs, q, Hkv, kt, vt).cpu().numpy()
    w = _check_all(out, host, wl.arrays["q"].astype(np.float64), wl.arrays["k"].reshape(B * Hkv, N, 128).astype(np.float64),
                   wl.arrays["v"].reshape(B * Hkv, N, 128).astype(np.float64), B, Hkv, Hq, tail)
    print("worst relative error", w)


def test_segments_reject_value_quantizers_with_different_rotations():
    gk, _ = _pair(128, 3, 0)
    gv1, _ = _pair(128, 3, 1)
    gv2, _ = _pair(128, 2, 2)
    x = torch.randn(1, 64, 128, device=_dev())
    kc, kn, kg = tq.tq_encode(gk, tq.TQ_PROD, x)
    v1 = tq.tq_encode(gv1, tq.TQ_MSE, x)
    v2 = tq.tq_encode(gv2, tq.TQ_MSE, x)
    segs = [tq.Segment(gk, gv1, kc, kn, kg, v1[0], v1[1], 64), tq.Segment(gk, gv2, kc, kn, kg, v2[0], v2[1], 64)]
    with pytest.raises(tq.TQError):
        tq.tq_attend_decode_segments(segs, torch.randn(1, 4, 128, device=_dev()), 1)


@pytest.mark.parametrize("mode,b_from,b_to,seed_to,nseq,n", [
    (tq.TQ_PROD, 4, 2, 0, 3, 1000), (tq.TQ_PROD, 3, 2, 7, 2, 777), (tq.TQ_MSE, 4, 2, 1, 4, 1000),
    (tq.TQ_MSE, 3, 1, 9, 2, 333), (tq.TQ_MSE_KEYS, 4, 3, 0, 2, 500)])
def test_requantize_matches_oracle(mode, b_from, b_to, seed_to, nseq, n):
    """Codes of the older width re-encoded at the newer one: the GPU's output
    against the oracle's encoding of its float64 decode of the GPU's input
    codes (same or different seed, hence same or different Pi)."""
    print(f"case: requantize mode={mode} {b_from} -> {b_to} bits seed_to={seed_to} nseq={nseq} n={n}", flush=True)
    seed_from = 1 if mode == tq.TQ_MSE else 0
    gf, of = _pair(128, b_from, seed_from)
    gt, ot = _pair(128, b_to, seed_to)
    x = torch.from_numpy(np.random.default_rng(n).standard_normal((nseq, n, 128)).astype(np.float32) * 2).to(_dev())
    c, nn, gg = tq.tq_encode(gf, mode, x)
    c2, n2, g2 = tq.tq_requantize(gf, gt, mode, c, nn, gg, nseq, n)
    torch.cuda.synchronize()
    cw, cw2 = P.to_u32(c), P.to_u32(c2)
    nn, n2 = nn.cpu().numpy().astype(np.float64), n2.cpu().numpy()
    per, per2 = gf.code_words(mode, 1, n), gt.code_words(mode, 1, n)
    for s in range(nseq):
        sl = slice(s * n, (s + 1) * n)
        if mode == tq.TQ_PROD:
            i, b = o.unpack_prod(cw[s * per:(s + 1) * per].reshape(n, -1), b_from - 1, 128)
            xd = o.decode_prod(of, i, b, nn[sl], gg.cpu().numpy().astype(np.float64)[sl])
            P.check_prod_codes(ot, xd, cw2[s * per2:(s + 1) * per2], n2[sl], g2.cpu().numpy()[sl])
        elif mode == tq.TQ_MSE:
            i = o.unpack_mse(cw[s * per:(s + 1) * per], n, b_from, 128)
            xd = o.decode_mse(of, i, nn[sl])
            P.check_mse_codes(ot, xd, cw2[s * per2:(s + 1) * per2], n2[sl])
        else:
            i = o.unpack_mse_keys(cw[s * per:(s + 1) * per].reshape(n, -1), b_from, 128)
            xd = o.decode_mse(of, i, nn[sl])
            P.check_mse_key_codes(ot, xd, cw2[s * per2:(s + 1) * per2], n2[sl])
