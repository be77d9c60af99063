"""GPU parity for MSE-only keys (all b bits to the Lloyd-Max index, no QJL
plane): tq_encode / tq_decode with TQ_MSE_KEYS, then tq_scores (logits and
top-k) and tq_attend_decode on a quantizer switched to that key mode, each
against the oracle on the GPU's own codes (tolerances in tests/parity.py)."""
import math

import numpy as np
import pytest

from oracle import tq_oracle as o
from tests import parity as P
from vector_quantization_tq_amd import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from vector_quantization_tq_amd import tq  # noqa: E402


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def _pair(d, bits, seed=0):
    """A fresh quantizer in MSE-key mode (the key mode is per-quantizer state,
    so these are not shared with the prod-key tests) and its oracle twin."""
    g = tq.Quantizer(d, bits, seed)
    g.set_key_mode(tq.TQ_MSE_KEYS)
    return g, o.Quantizer(d, bits, seed)


def _keys(rng, nseq, n, d):
    # anisotropic channels, as in the other key tests
    return (rng.standard_normal((nseq, n, d)) * np.exp(rng.uniform(0, math.log(50), (nseq, 1, d)))).astype(np.float32)


def _encode(g, x_t):
    codes, norms, gam = tq.tq_encode(g, tq.TQ_MSE_KEYS, x_t)
    assert gam is None
    torch.cuda.synchronize()
    return codes, norms


@pytest.mark.parametrize("d,bits,nseq,n,bf16", [
    (128, 4, 2, 1000, True), (128, 3, 1, 777, False), (128, 2, 3, 64, True), (128, 1, 1, 130, False),
    (96, 4, 1, 65, False), (16, 2, 2, 33, False), (48, 3, 1, 100, True), (200, 4, 1, 300, False),
    (200, 2, 1, 70, True), (3, 4, 1, 10, False)])
def test_encode_mse_keys_shapes(d, bits, nseq, n, bf16):
    print(f"case: mse keys encode d={d} bits={bits} nseq={nseq} n={n} bf16={bf16}", flush=True)
    rng = np.random.default_rng(d * 10 + bits)
    g, oq = _pair(d, bits)
    xt = torch.from_numpy(_keys(rng, nseq, n, d)).to(_dev())
    if bf16:
        xt = xt.bfloat16()
    codes, norms = _encode(g, xt)
    xs = xt.float().cpu().numpy().astype(np.float64).reshape(nseq * n, d)
    N = nseq * n
    assert g.code_words(tq.TQ_MSE_KEYS, nseq, n) == N * ((d + 31) // 32) * bits
    cw = P.to_u32(codes)[: g.code_words(tq.TQ_MSE_KEYS, nseq, n)]
    _, st = P.check_mse_key_codes(oq, xs, cw, norms.cpu().numpy()[:N])
    print(st)


def test_encode_mse_keys_zero_vector_and_decode():
    print("case: mse keys zero vector + decode d=128 bits=3", flush=True)
    rng = np.random.default_rng(3)
    g, oq = _pair(128, 3)
    x = rng.standard_normal((300, 128)).astype(np.float32) * 2
    x[7] = 0.0
    xt = torch.from_numpy(x).to(_dev())
    codes, norms = _encode(g, xt)
    cw = P.to_u32(codes)[: g.code_words(tq.TQ_MSE_KEYS, 1, 300)]
    idx, _ = P.check_mse_key_codes(oq, x.astype(np.float64), cw, norms.cpu().numpy()[:300])
    assert np.all(idx[7] == 3) and norms[7].item() == 0.0   # y = 0 -> index K/2 - 1
    dec = tq.tq_decode(g, tq.TQ_MSE_KEYS, codes, norms, None, 1, 300)[0].cpu().numpy()
    ref = o.decode_mse(oq, idx, norms.cpu().numpy()[:300].astype(np.float64))
    nz = np.linalg.norm(ref, axis=1) > 0
    err = np.abs(dec[nz] - ref[nz]).max(axis=1) / np.linalg.norm(ref[nz], axis=1)
    assert err.max() < 1e-5 and np.all(dec[~nz] == 0)


def _scores_case(d, bits, B, Hkv, Hq, n, bf16, seed=0, topk=0):
    rng = np.random.default_rng(seed)
    g, oq = _pair(d, bits)
    kt = torch.from_numpy(_keys(rng, B * Hkv, n, d)).to(_dev())
    qt = torch.from_numpy(rng.standard_normal((B, Hq, d)).astype(np.float32)).to(_dev())
    if bf16:
        kt, qt = kt.bfloat16(), qt.bfloat16()
    codes, norms = _encode(g, kt)
    logits = tq.tq_scores(g, qt, codes, norms, None, Hkv, n)
    if topk:
        s, i = tq.tq_scores(g, qt, codes, norms, None, Hkv, n, topk=topk)
        s, i = s.cpu().numpy(), i.cpu().numpy()
    logits = logits.cpu().numpy()
    cw = P.to_u32(codes)
    nn = norms.cpu().numpy().astype(np.float64)
    qs = qt.float().cpu().numpy().astype(np.float64)
    G = Hq // Hkv
    per = g.code_words(tq.TQ_MSE_KEYS, 1, n)
    worst = 0.0
    for b in range(B):
        for h in range(Hkv):
            sq = b * Hkv + h
            hs = slice(h * G, (h + 1) * G)
            idx = o.unpack_mse_keys(cw[sq * per:(sq + 1) * per].reshape(n, -1), bits, d)
            kn = nn[sq * n:(sq + 1) * n]
            ref = o.scores_mse(oq, qs[b, hs], idx, kn)
            worst = max(worst, P.check_logits(logits[b, hs], ref, np.linalg.norm(qs[b, hs], axis=1), kn, d))
            if topk:
                P.check_topk(s[b, hs], i[b, hs], ref, np.linalg.norm(qs[b, hs], axis=1), kn, d)
                # exact selection over the GPU's own logits
                for r in range(G):
                    order = np.lexsort((np.arange(n), -logits[b, h * G + r].astype(np.float64)))[:topk]
                    assert np.array_equal(order, i[b, h * G + r])
    return worst


@pytest.mark.parametrize("d,bits,B,Hkv,Hq,n,bf16", [
    (128, 4, 2, 2, 8, 1000, True), (128, 3, 1, 4, 4, 777, False), (128, 2, 1, 2, 14, 4099, True),
    (128, 1, 1, 1, 3, 200, False), (200, 4, 1, 1, 5, 3000, False), (64, 3, 2, 1, 2, 65, False),
    (16, 2, 1, 1, 1, 5, False)])
def test_scores_mse_keys(d, bits, B, Hkv, Hq, n, bf16):
    print(f"case: mse keys scores d={d} bits={bits} B={B} Hkv={Hkv} Hq={Hq} n={n}", flush=True)
    print("worst", _scores_case(d, bits, B, Hkv, Hq, n, bf16, seed=d + bits))


@pytest.mark.parametrize("d,bits,Hq,n,topk", [(128, 4, 8, 5000, 10), (200, 3, 20, 20000, 32), (64, 2, 3, 100, 7)])
def test_topk_mse_keys(d, bits, Hq, n, topk):
    print(f"case: mse keys top-k d={d} bits={bits} Hq={Hq} n={n} k={topk}", flush=True)
    _scores_case(d, bits, 1, 1, Hq, n, False, seed=5, topk=topk)


def test_scores_prep_matches_for_mse_keys():
    """tq_query_prep + tq_scores_from_prep equals tq_scores bit for bit."""
    print("case: mse keys prep + scan", flush=True)
    rng = np.random.default_rng(9)
    g, _ = _pair(128, 4)
    kt = torch.from_numpy(_keys(rng, 2, 513, 128)).to(_dev())
    qt = torch.from_numpy(rng.standard_normal((1, 8, 128)).astype(np.float32)).to(_dev())
    codes, norms = _encode(g, kt)
    a = tq.tq_scores(g, qt, codes, norms, None, 2, 513)
    ws = tq.tq_query_prep(g, qt, 2)
    b = tq.tq_scores_from_prep(g, 1, 8, 2, codes, norms, None, 513, ws)
    assert torch.equal(a, b)


def _bf16(u16):
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).to(_dev()).view(torch.bfloat16)


@pytest.mark.parametrize("d,B,Hkv,Hq,N,tail,kbits,vbits", [
    (128, 1, 2, 8, 1000, 0, 4, 4), (128, 2, 2, 8, 777, 37, 3, 3), (128, 1, 1, 6, 300, 5, 2, 4),
    (128, 1, 2, 2, 129, 0, 1, 2), (128, 1, 8, 32, 4096, 256, 4, 3), (64, 1, 2, 8, 2000, 10, 3, 2),
    (96, 1, 2, 8, 2000, 0, 3, 3), (96, 1, 2, 4, 700, 3, 1, 4), (256, 1, 2, 8, 3000, 64, 4, 4)])
def test_attend_mse_keys(d, B, Hkv, Hq, N, tail, kbits, vbits):
    print(f"case: mse keys attend d={d} B={B} Hkv={Hkv} Hq={Hq} N={N} tail={tail} K{kbits} V{vbits}", flush=True)
    rng = np.random.default_rng(N + kbits)
    a = W._gqa_tensors(rng, B, Hkv, Hq, N, d)
    k = _bf16(a["k_bf16"]).view(B * Hkv, N, d)
    v = _bf16(a["v_bf16"]).view(B * Hkv, N, d)
    q = _bf16(a["q_bf16"])
    n_comp = N - tail
    gk, ok = _pair(d, kbits, 0)
    gv, ov = tq.Quantizer(d, vbits, 1), o.Quantizer(d, vbits, 1)
    kc, vc = k[:, :n_comp].contiguous(), v[:, :n_comp].contiguous()
    kcodes, kn = _encode(gk, kc)
    vcodes, vn, _ = tq.tq_encode(gv, tq.TQ_MSE, vc)
    kt = k[:, n_comp:].contiguous().view(B, Hkv, tail, d) if tail else None
    vt = v[:, n_comp:].contiguous().view(B, Hkv, tail, d) if tail else None
    out = tq.tq_attend_decode(gk, gv, q, kcodes, kn, None, vcodes, vn, Hkv, n_comp, kt, vt).cpu().numpy()
    G = Hq // Hkv
    kw, vw = P.to_u32(kcodes), P.to_u32(vcodes)
    kn, vn = kn.cpu().numpy().astype(np.float64), vn.cpu().numpy().astype(np.float64)
    qs = q.float().cpu().numpy().astype(np.float64)
    kf, vf = k.float().cpu().numpy().astype(np.float64), v.float().cpu().numpy().astype(np.float64)
    perk, perv = gk.code_words(tq.TQ_MSE_KEYS, 1, n_comp), gv.code_words(tq.TQ_MSE, 1, n_comp)
    worst = 0.0
    groups = [(b, h) for b in range(B) for h in range(Hkv)][:4]
    for (b, h) in groups:
        s = b * Hkv + h
        ki = o.unpack_mse_keys(kw[s * perk:(s + 1) * perk].reshape(n_comp, -1), kbits, d)
        vi = o.unpack_mse(vw[s * perv:(s + 1) * perv], n_comp, vbits, d)
        sl = slice(s * n_comp, (s + 1) * n_comp)
        ref = o.attend(ok, ov, qs[b, h * G:(h + 1) * G], ki, None, kn[sl], None, vi, vn[sl],
                       kf[s, n_comp:] if tail else None, vf[s, n_comp:] if tail else None)
        worst = max(worst, P.check_attention(out[b, h * G:(h + 1) * G], ref))
    print("worst relative error", worst)


def test_key_mode_errors():
    """Prod keys need bits >= 2; the key mode must be one of the two; with
    prod keys the gammas are required."""
    print("case: key mode errors", flush=True)
    g1 = tq.Quantizer(128, 1, 0)
    with pytest.raises(tq.TQError):
        g1.set_key_mode(tq.TQ_PROD)
    g1.set_key_mode(tq.TQ_MSE_KEYS)
    with pytest.raises(tq.TQError):
        g1.set_key_mode(tq.TQ_MSE)
    g = tq.Quantizer(128, 3, 0)
    kt = torch.randn(1, 64, 128, device=_dev())
    qt = torch.randn(1, 2, 128, device=_dev())
    codes, norms, gam = tq.tq_encode(g, tq.TQ_PROD, kt)
    with pytest.raises((tq.TQError, ValueError)):   # the binding refuses it before the library does
        tq.tq_scores(g, qt, codes, norms, None, 1, 64)
    # 1-bit MSE keys score without a prod codebook
    c1, n1 = _encode(g1, kt)
    assert torch.isfinite(tq.tq_scores(g1, qt, c1, n1, None, 1, 64)).all()
