"""GPU parity for quantizers with the structured rotation Pi = H D / sqrt(d)
(tq_make_quantizer_ex with TQ_ROT_HADAMARD): encode (keys and values),
decode, logits, top-k and decode attention through the C ABI against the
oracle built with the same rotation (tolerances in tests/parity.py)."""
import math

import numpy as np
import pytest

from oracle import tq_oracle as o
from tests import parity as P
from vector_quantization_tq_amd import workloads as W

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
        _QZ[key] = (tq.Quantizer(d, bits, seed, rotation=tq.TQ_ROT_HADAMARD),
                    o.Quantizer(d, bits, seed, rotation_kind="hadamard"))
    return _QZ[key]


def _keys(rng, nseq, n, d):
    return (rng.standard_normal((nseq, n, d)) * np.exp(rng.uniform(0, math.log(50), (nseq, 1, d)))).astype(np.float32)


@pytest.mark.parametrize("d,bits,nseq,n,bf16", [
    (128, 3, 2, 1000, True), (128, 4, 1, 777, False), (64, 2, 1, 300, True), (256, 3, 1, 200, False),
    (16, 2, 2, 65, False),
    (128, 2, 3, 20011, False)])   # fp32 keys over several tiles per workgroup of the persistent grid
def test_encode_prod_hadamard(d, bits, nseq, n, bf16):
    print(f"case: hadamard prod encode d={d} bits={bits} nseq={nseq} n={n}", flush=True)
    g, oq = _pair(d, bits)
    xt = torch.from_numpy(_keys(np.random.default_rng(d + bits), nseq, n, d)).to(_dev())
    if bf16:
        xt = xt.bfloat16()
    codes, norms, gam = tq.tq_encode(g, tq.TQ_PROD, xt)
    torch.cuda.synchronize()
    N = nseq * n
    xs = xt.float().cpu().numpy().astype(np.float64).reshape(N, d)
    _, _, st = P.check_prod_codes(oq, xs, P.to_u32(codes)[: g.code_words(tq.TQ_PROD, nseq, n)],
                                  norms.cpu().numpy()[:N], gam.cpu().numpy()[:N])
    print(st)


@pytest.mark.parametrize("d,bits,n", [(128, 3, 1000), (128, 4, 4101), (32, 1, 70)])
def test_encode_mse_and_decode_hadamard(d, bits, n):
    print(f"case: hadamard mse encode + decode d={d} bits={bits} n={n}", flush=True)
    g, oq = _pair(d, bits)
    x = np.random.default_rng(n).standard_normal((n, d)).astype(np.float32)
    xt = torch.from_numpy(x).to(_dev())
    codes, norms, _ = tq.tq_encode(g, tq.TQ_MSE, xt)
    dec = tq.tq_decode(g, tq.TQ_MSE, codes, norms, None, 1, n)[0].cpu().numpy()
    idx, _ = P.check_mse_codes(oq, x.astype(np.float64), P.to_u32(codes), norms.cpu().numpy())
    ref = o.decode_mse(oq, idx, norms.cpu().numpy().astype(np.float64))
    err = np.abs(dec - ref).max(axis=1) / np.linalg.norm(ref, axis=1)
    assert err.max() < 1e-5


@pytest.mark.parametrize("d,bits,B,Hkv,Hq,n,topk", [
    (128, 3, 2, 2, 8, 1000, 0), (128, 4, 1, 4, 16, 3000, 0), (256, 2, 1, 1, 5, 500, 0), (128, 3, 1, 1, 10, 5000, 10)])
def test_scores_hadamard(d, bits, B, Hkv, Hq, n, topk):
    print(f"case: hadamard scores d={d} bits={bits} B={B} Hkv={Hkv} Hq={Hq} n={n} k={topk}", flush=True)
    rng = np.random.default_rng(d * bits + n)
    g, oq = _pair(d, bits)
    kt = torch.from_numpy(_keys(rng, B * Hkv, n, d)).to(_dev()).bfloat16()
    qt = torch.from_numpy(rng.standard_normal((B, Hq, d)).astype(np.float32)).to(_dev())
    codes, norms, gam = tq.tq_encode(g, tq.TQ_PROD, kt)
    logits = tq.tq_scores(g, qt, codes, norms, gam, Hkv, n).cpu().numpy()
    if topk:
        s, i = tq.tq_scores(g, qt, codes, norms, gam, Hkv, n, topk=topk)
        s, i = s.cpu().numpy(), i.cpu().numpy()
    cw = P.to_u32(codes)
    nn, gg = norms.cpu().numpy().astype(np.float64), gam.cpu().numpy().astype(np.float64)
    qs = qt.cpu().numpy().astype(np.float64)
    G, per = Hq // Hkv, g.code_words(tq.TQ_PROD, 1, n)
    for b in range(B):
        for h in range(Hkv):
            sq, hs = b * Hkv + h, slice(h * (Hq // Hkv), (h + 1) * (Hq // Hkv))
            idx, bits01 = o.unpack_prod(cw[sq * per:(sq + 1) * per].reshape(n, -1), bits - 1, d)
            kn = nn[sq * n:(sq + 1) * n]
            ref = o.scores(oq, qs[b, hs], idx, bits01, kn, gg[sq * n:(sq + 1) * n])
            P.check_logits(logits[b, hs], ref, np.linalg.norm(qs[b, hs], axis=1), kn, d)
            if topk:
                P.check_topk(s[b, hs], i[b, hs], ref, np.linalg.norm(qs[b, hs], axis=1), kn, d)


@pytest.mark.parametrize("B,Hkv,Hq,N,tail,bits", [(1, 2, 8, 1000, 0, 3), (2, 2, 8, 777, 37, 4)])
def test_attend_hadamard(B, Hkv, Hq, N, tail, bits):
    print(f"case: hadamard attend B={B} Hkv={Hkv} Hq={Hq} N={N} tail={tail} bits={bits}", flush=True)
    d = 128
    a = W._gqa_tensors(np.random.default_rng(N + bits), B, Hkv, Hq, N, d)

    def bf(u16):
        return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).to(_dev()).view(torch.bfloat16)

    k, v, q = bf(a["k_bf16"]).view(B * Hkv, N, d), bf(a["v_bf16"]).view(B * Hkv, N, d), bf(a["q_bf16"])
    n_comp = N - tail
    gk, ok = _pair(d, bits, 0)
    gv, ov = _pair(d, bits, 1)
    kcodes, kn, kg = tq.tq_encode(gk, tq.TQ_PROD, k[:, :n_comp].contiguous())
    vcodes, vn, _ = tq.tq_encode(gv, tq.TQ_MSE, v[:, :n_comp].contiguous())
    kt = k[:, n_comp:].contiguous().view(B, Hkv, tail, d) if tail else None
    vt = v[:, n_comp:].contiguous().view(B, Hkv, tail, d) if tail else None
    out = tq.tq_attend_decode(gk, gv, q, kcodes, kn, kg, vcodes, vn, Hkv, n_comp, kt, vt).cpu().numpy()
    G = Hq // Hkv
    kw, vw = P.to_u32(kcodes), P.to_u32(vcodes)
    kn, kg, vn = (t.cpu().numpy().astype(np.float64) for t in (kn, kg, vn))
    qs = q.float().cpu().numpy().astype(np.float64)
    kf, vf = k.float().cpu().numpy().astype(np.float64), v.float().cpu().numpy().astype(np.float64)
    perk, perv = gk.code_words(tq.TQ_PROD, 1, n_comp), gv.code_words(tq.TQ_MSE, 1, n_comp)
    for b in range(B):
        for h in range(Hkv):
            s = b * Hkv + h
            ki, kb = o.unpack_prod(kw[s * perk:(s + 1) * perk].reshape(n_comp, -1), bits - 1, d)
            vi = o.unpack_mse(vw[s * perv:(s + 1) * perv], n_comp, bits, d)
            sl = slice(s * n_comp, (s + 1) * n_comp)
            ref = o.attend(ok, ov, qs[b, h * G:(h + 1) * G], ki, kb, kn[sl], kg[sl], vi, vn[sl],
                           kf[s, n_comp:] if tail else None, vf[s, n_comp:] if tail else None)
            P.check_attention(out[b, h * G:(h + 1) * G], ref)


@pytest.mark.parametrize("mode", ["prod", "mse", "mse_keys"])
def test_encode_hadamard_gqa_layer_multi_tile(mode):
    """Keys (prod and MSE-only) and values of 8 (batch, KV head) sequences of
    the GQA decode layer (bf16, 32768 tokens each) under the Hadamard rotation:
    the d = 128 encoder with the exact +-1 rotation operand, many tiles per
    persistent workgroup; every code of every sequence is checked."""
    print(f"case: hadamard GQA-layer encode {mode} 8 x 32768", flush=True)
    rng = np.random.default_rng(33)
    a = W._gqa_tensors(rng, 1, 8, 32, 32768, 128)
    key = "v_bf16" if mode == "mse" else "k_bf16"
    xt = torch.from_numpy(np.ascontiguousarray(a[key]).view(np.int16)).to(_dev()).view(torch.bfloat16).view(8, 32768, 128)
    xs = a[key[0]].reshape(8, 32768, 128).astype(np.float64)
    g, oq = _pair(128, 3)
    m = {"prod": tq.TQ_PROD, "mse": tq.TQ_MSE, "mse_keys": tq.TQ_MSE_KEYS}[mode]
    codes, norms, gam = tq.tq_encode(g, m, xt)
    torch.cuda.synchronize()
    cw = P.to_u32(codes)
    per = g.code_words(m, 1, 32768)
    nn = norms.cpu().numpy()
    gg = gam.cpu().numpy() if gam is not None else None
    for s in range(8):
        sl = slice(s * 32768, (s + 1) * 32768)
        c = cw[s * per:(s + 1) * per]
        if mode == "prod":
            P.check_prod_codes(oq, xs[s], c, nn[sl], gg[sl])
        elif mode == "mse":
            P.check_mse_codes(oq, xs[s], c, nn[sl])
        else:
            P.check_mse_key_codes(oq, xs[s], c, nn[sl])


@pytest.mark.parametrize("d,bits,nseq,n,bf16,mode", [
    (128, 3, 3, 1000, True, "mse"), (128, 4, 2, 4101, False, "mse"), (128, 2, 2, 777, True, "mse_keys"),
    (128, 1, 1, 300, True, "mse"), (64, 3, 2, 333, True, "mse"), (64, 4, 1, 129, False, "mse_keys"),
    (32, 2, 2, 65, True, "mse"), (32, 3, 1, 100, False, "mse_keys"), (256, 3, 2, 1000, True, "mse"),
    (256, 4, 1, 97, False, "mse"), (256, 2, 2, 33, True, "mse_keys"), (256, 1, 1, 64, False, "mse_keys"),
    (128, 3, 1, 1, True, "mse"), (256, 3, 1, 1, True, "mse_keys")])
def test_encode_walsh_hadamard_butterfly(d, bits, nseq, n, bf16, mode):
    """Values and MSE-only keys under the Hadamard rotation take the
    butterfly encoder (the fast Walsh-Hadamard transform in registers, one
    token per lane, two lanes per token at d = 256): every code of every
    sequence against the oracle, ragged tails (tiles of 64 tokens, 32 at
    d = 256), bf16 and float input.  The first vector of each sequence is
    zero (every coordinate of H D x exactly 0: the cell below the middle
    threshold, as the oracle takes it)."""
    print(f"case: hadamard butterfly encode {mode} d={d} bits={bits} nseq={nseq} n={n} bf16={bf16}", flush=True)
    g, oq = _pair(d, bits)
    x = _keys(np.random.default_rng(d * 10 + bits + n), nseq, n, d)
    x[:, 0] = 0.0
    xt = torch.from_numpy(x).to(_dev())
    if bf16:
        xt = xt.bfloat16()
    m = tq.TQ_MSE if mode == "mse" else tq.TQ_MSE_KEYS
    codes, norms, _ = tq.tq_encode(g, m, xt)
    torch.cuda.synchronize()
    xs = xt.float().cpu().numpy().astype(np.float64)
    cw = P.to_u32(codes)
    per = g.code_words(m, 1, n)
    nn = norms.cpu().numpy()
    for s in range(nseq):
        c = cw[s * per:(s + 1) * per]
        if mode == "mse":
            P.check_mse_codes(oq, xs[s], c, nn[s * n:(s + 1) * n])
        else:
            P.check_mse_key_codes(oq, xs[s], c, nn[s * n:(s + 1) * n])
