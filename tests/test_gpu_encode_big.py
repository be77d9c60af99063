"""GPU parity for 256 < d <= 1024: the general tile encoder (16-key and
32-value tiles) and the vector-ALU logits scan, against the oracle on
identical inputs and codes; ragged tails, both input types, d not a multiple
of 32; top-k above d = 256 is refused."""
import math

import numpy as np
import pytest

from oracle import tq_oracle as o
from tests import parity as P

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from vector_quantization_tq_amd import tq  # noqa: E402

_QZ = {}


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def _pair(d, bits, seed=0):
    key = (d, bits, seed)
    if key not in _QZ:
        _QZ[key] = (tq.Quantizer(d, bits, seed), o.Quantizer(d, bits, seed))
    return _QZ[key]


def _data(rng, nseq, n, d):
    # per-channel scales log-uniform over [1, 50], as the decode-layer keys
    return (rng.standard_normal((nseq, n, d)) * np.exp(rng.uniform(0, math.log(50), (nseq, 1, d)))).astype(np.float32)


@pytest.mark.parametrize("d,bits,mode,nseq,n,bf16", [
    (300, 3, "prod", 2, 203, False), (512, 4, "prod", 1, 130, True), (1024, 3, "prod", 1, 70, False),
    (257, 2, "prod", 2, 33, True),
    (300, 3, "mse", 2, 100, True), (1024, 4, "mse", 1, 64, False), (520, 2, "mse", 1, 31, False),
    (384, 4, "mse_keys", 2, 90, False), (1000, 3, "mse_keys", 1, 17, True)])
def test_big_encoder(d, bits, mode, nseq, n, bf16):
    print(f"case: encoder d={d} bits={bits} {mode} nseq={nseq} n={n} bf16={bf16}", flush=True)
    rng = np.random.default_rng(d + bits)
    g, oq = _pair(d, bits)
    x = _data(rng, nseq, n, d)
    xt = torch.from_numpy(x).to(_dev())
    if bf16:
        xt = xt.bfloat16()
    m = {"prod": tq.TQ_PROD, "mse": tq.TQ_MSE, "mse_keys": tq.TQ_MSE_KEYS}[mode]
    codes, norms, gam = tq.tq_encode(g, m, xt)
    torch.cuda.synchronize()
    xs = xt.float().cpu().numpy().astype(np.float64)
    cw = P.to_u32(codes)
    per = g.code_words(m, 1, n)
    nn = norms.cpu().numpy()
    for s in range(nseq):
        sl = slice(s * n, (s + 1) * n)
        c = cw[s * per:(s + 1) * per]
        if mode == "prod":
            P.check_prod_codes(oq, xs[s], c, nn[sl], gam.cpu().numpy()[sl])
        elif mode == "mse":
            P.check_mse_codes(oq, xs[s], c, nn[sl])
        else:
            P.check_mse_key_codes(oq, xs[s], c, nn[sl])


@pytest.mark.parametrize("d,bits,B,Hkv,Hq,n,mse_keys", [
    (300, 3, 1, 2, 6, 333, False), (1024, 4, 1, 1, 5, 257, False), (640, 2, 2, 1, 3, 100, False),
    (1024, 3, 1, 1, 2, 120, True), (272, 4, 1, 2, 10, 77, True)])
def test_big_logits(d, bits, B, Hkv, Hq, n, mse_keys):
    """Logits at 256 < d <= 1024 against the oracle's scorer on the GPU's own
    codes; G = Hq / Hkv covers one and several passes of 4 queries."""
    print(f"case: logits d={d} bits={bits} B={B} Hkv={Hkv} Hq={Hq} n={n} mse_keys={mse_keys}", flush=True)
    rng = np.random.default_rng(7 * d + bits)
    g = tq.Quantizer(d, bits, 3)
    oq = o.Quantizer(d, bits, 3)
    if mse_keys:
        g.set_key_mode(tq.TQ_MSE_KEYS)
    mode = tq.TQ_MSE_KEYS if mse_keys else tq.TQ_PROD
    kt = torch.from_numpy(_data(rng, B * Hkv, n, d)).to(_dev())
    qt = torch.from_numpy(rng.standard_normal((B, Hq, d)).astype(np.float32)).to(_dev())
    codes, norms, gam = tq.tq_encode(g, mode, kt)
    logits = tq.tq_scores(g, qt, codes, norms, None if mse_keys else gam, Hkv, n).cpu().numpy()
    cw = P.to_u32(codes)
    nn = norms.cpu().numpy().astype(np.float64)
    gg = None if mse_keys else gam.cpu().numpy().astype(np.float64)
    qs = qt.cpu().numpy().astype(np.float64)
    G = Hq // Hkv
    per = g.code_words(mode, 1, n)
    worst = 0.0
    for b in range(B):
        for h in range(Hkv):
            s = b * Hkv + h
            hs = slice(h * G, (h + 1) * G)
            kn = nn[s * n:(s + 1) * n]
            if mse_keys:
                idx = o.unpack_mse_keys(cw[s * per:(s + 1) * per].reshape(n, -1), bits, d)
                ref = o.scores_mse(oq, qs[b, hs], idx, kn)
            else:
                idx, bits01 = o.unpack_prod(cw[s * per:(s + 1) * per].reshape(n, -1), bits - 1, d)
                ref = o.scores(oq, qs[b, hs], idx, bits01, kn, gg[s * n:(s + 1) * n])
            worst = max(worst, P.check_logits(logits[b, hs], ref, np.linalg.norm(qs[b, hs], axis=1), kn, d))
    print("worst relative logit error", worst)


def test_big_topk_refused():
    print("case: top-k at d = 300 refused", flush=True)
    g, _ = _pair(300, 3)
    x = torch.randn(1, 64, 300, device=_dev())
    codes, norms, gam = tq.tq_encode(g, tq.TQ_PROD, x)
    q = torch.randn(1, 2, 300, device=_dev())
    with pytest.raises(tq.TQError):
        tq.tq_scores(g, q, codes, norms, gam, 1, 64, topk=5)


@pytest.mark.parametrize("mode,d,bits,n", [(0, 300, 3, 40), (0, 1024, 4, 24), (1, 1024, 3, 40), (1, 520, 2, 33)])
def test_big_decode(mode, d, bits, n):
    """tq_decode of codes written by the d > 256 encoder, against the
    oracle's decode of the same codes."""
    print(f"case: decode mode={mode} d={d} bits={bits} n={n}", flush=True)
    rng = np.random.default_rng(5 * d + bits)
    g, oq = _pair(d, bits)
    x = torch.from_numpy(rng.standard_normal((n, d)).astype(np.float32) * 3).to(_dev())
    codes, norms, gam = tq.tq_encode(g, mode, x)
    dec = tq.tq_decode(g, mode, codes, norms, gam, 1, n)[0].cpu().numpy()
    cw = P.to_u32(codes)
    nn = norms.cpu().numpy()[:n].astype(np.float64)
    if mode == 0:
        idx, bits01 = o.unpack_prod(cw[: g.code_words(0, 1, n)].reshape(n, -1), bits - 1, d)
        ref = o.decode_prod(oq, idx, bits01, nn, gam.cpu().numpy()[:n].astype(np.float64))
    else:
        idx = o.unpack_mse(cw, n, bits, d)
        ref = o.decode_mse(oq, idx, nn)
    err = np.abs(dec - ref).max(axis=1) / np.linalg.norm(ref, axis=1)
    assert err.max() < 1e-5, err.max()
