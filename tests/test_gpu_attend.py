"""GPU parity: tq_attend_decode through the C ABI against the oracle's
attention on the same codes (the GPU's packed keys and values fed to the
oracle), per output row |gpu - oracle| <= 1e-3 max(|oracle_e|, ||oracle_row||/sqrt(d))."""
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


def _pair(d, bits, seed):
    key = (d, bits, seed)
    if key not in _QZ:
        _QZ[key] = (tq.Quantizer(d, bits, seed), o.Quantizer(d, bits, seed))
    return _QZ[key]


def _dev():
    assert torch.cuda.is_available()
    return torch.device("cuda:0")


def _bf16(u16):
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).to(_dev()).view(torch.bfloat16)


def _run_case(k, v, q, B, Hkv, Hq, n_comp, n_tail, bits, scale=0.0, groups=None, kseed=0, vseed=1, vbits=None):
    """k, v: torch bf16 [B*Hkv, N, d]; q: torch [B, Hq, d]; bits for keys
    (vbits for values, default the same)."""
    d = k.shape[-1]
    vbits = bits if vbits is None else vbits
    gk, ok = _pair(d, bits, kseed)
    gv, ov = _pair(d, vbits, vseed)
    kc = k[:, :n_comp].contiguous()
    vc = v[:, :n_comp].contiguous()
    kcodes, kn, kg = tq.tq_encode(gk, tq.TQ_PROD, kc) if n_comp else (torch.empty(4, dtype=torch.int32, device=_dev()),
                                                                      torch.empty(4, device=_dev()),
                                                                      torch.empty(4, device=_dev()))
    vcodes, vn, _ = tq.tq_encode(gv, tq.TQ_MSE, vc) if n_comp else (torch.empty(4, dtype=torch.int32, device=_dev()),
                                                                    torch.empty(4, device=_dev()), None)
    kt = k[:, n_comp:].contiguous().view(B, Hkv, n_tail, d) if n_tail else None
    vt = v[:, n_comp:].contiguous().view(B, Hkv, n_tail, d) if n_tail else None
    out = tq.tq_attend_decode(gk, gv, q, kcodes, kn, kg, vcodes, vn, Hkv, n_comp, kt, vt, scale).cpu().numpy()
    G = Hq // Hkv
    kw = P.to_u32(kcodes)
    vw = P.to_u32(vcodes)
    kn = kn.cpu().numpy().astype(np.float64)
    kg = kg.cpu().numpy().astype(np.float64)
    vn = vn.cpu().numpy().astype(np.float64)
    qs = q.float().cpu().numpy().astype(np.float64)
    kf = k.float().cpu().numpy().astype(np.float64)
    vf = v.float().cpu().numpy().astype(np.float64)
    perk = gk.code_words(tq.TQ_PROD, 1, n_comp) if n_comp else 0
    perv = gv.code_words(tq.TQ_MSE, 1, n_comp) if n_comp else 0
    worst = 0.0
    todo = groups if groups is not None else [(b, h) for b in range(B) for h in range(Hkv)]
    for (b, h) in todo:
        s = b * Hkv + h
        if n_comp:
            ki, kb = o.unpack_prod(kw[s * perk:(s + 1) * perk].reshape(n_comp, -1), bits - 1, d)
            vi = o.unpack_mse(vw[s * perv:(s + 1) * perv], n_comp, vbits, d)
        else:
            ki = np.zeros((0, d), dtype=np.int64); kb = np.zeros((0, d), dtype=np.uint8); vi = ki
        sl = slice(s * n_comp, (s + 1) * n_comp)
        ref = o.attend(ok, ov, qs[b, h * G:(h + 1) * G], ki, kb, kn[sl], kg[sl], vi, vn[sl],
                       kf[s, n_comp:] if n_tail else None, vf[s, n_comp:] if n_tail else None,
                       scale=None if scale <= 0 else scale)
        worst = max(worst, P.check_attention(out[b, h * G:(h + 1) * G], ref))
    return worst


def _gqa_inputs(B, Hkv, Hq, N, d, seed):
    rng = np.random.default_rng(seed)
    a = W._gqa_tensors(rng, B, Hkv, Hq, N, d)
    k = _bf16(a["k_bf16"]).view(B * Hkv, N, d)
    v = _bf16(a["v_bf16"]).view(B * Hkv, N, d)
    q = _bf16(a["q_bf16"])
    return k, v, q


@pytest.mark.parametrize("B,Hkv,Hq,N,tail,bits,qf32", [
    (2, 2, 8, 1000, 0, 3, False), (1, 2, 8, 777, 37, 4, False), (1, 1, 1, 300, 0, 2, True),
    (1, 1, 6, 129, 5, 3, True), (1, 2, 2, 100, 100, 3, False), (1, 1, 4, 1, 0, 3, False),
    (2, 8, 32, 4096, 0, 3, False), (1, 8, 32, 8192, 256, 4, False)])
def test_attend_shapes(B, Hkv, Hq, N, tail, bits, qf32):
    print(f"case: attend B={B} Hkv={Hkv} Hq={Hq} N={N} tail={tail} bits={bits}", flush=True)
    k, v, q = _gqa_inputs(B, Hkv, Hq, N, 128, seed=N + tail)
    if qf32:
        q = q.float()
    w = _run_case(k, v, q, B, Hkv, Hq, N - tail, tail, bits)
    print("worst relative error", w)


@pytest.mark.parametrize("d,B,Hkv,Hq,N,tail,bits,vbits", [
    (64, 2, 2, 8, 1000, 0, 3, 3), (64, 1, 8, 32, 9000, 256, 4, 2), (64, 1, 1, 1, 300, 0, 2, 4),
    (96, 1, 2, 8, 1000, 37, 3, 3), (96, 2, 4, 16, 5000, 0, 4, 4), (96, 1, 1, 6, 129, 5, 2, 1),
    (256, 1, 2, 8, 1000, 0, 3, 3), (256, 1, 4, 16, 6000, 300, 4, 4), (256, 1, 1, 4, 200, 0, 2, 2),
    (256, 1, 8, 32, 20000, 0, 3, 4)])
def test_attend_head_dims(d, B, Hkv, Hq, N, tail, bits, vbits):
    """Head dimensions 64, 96 and 256: keys in 1, 2 or 3 groups of a 128-wide
    MFMA chunk (96 leaves one lane group on zero operands) or two chunks
    (256); 16-coordinate value tiles spread over the waves (96: the last wave
    has none); key rows of 6 or 9 words (not 16-byte runs) staged by 4-byte
    copies; ragged tails up to 300 tokens (past the merge's first rounds)."""
    print(f"case: attend d={d} B={B} Hkv={Hkv} Hq={Hq} N={N} tail={tail} K{bits} V{vbits}", flush=True)
    k, v, q = _gqa_inputs(B, Hkv, Hq, N, d, seed=d + N + tail)
    groups = [(b, h) for b in range(B) for h in range(Hkv)][:3]
    w = _run_case(k, v, q, B, Hkv, Hq, N - tail, tail, bits, vbits=vbits, groups=groups)
    print("worst relative error", w)


def test_attend_head_dim_errors():
    """Unsupported head dimensions and sparse V outside d = 128 are refused."""
    print("case: attend head-dim errors", flush=True)
    for d in (32, 192):
        k, v, q = _gqa_inputs(1, 1, 4, 64, d, seed=d)
        g = tq.Quantizer(d, 3, 0)
        kc, kn, kg = tq.tq_encode(g, tq.TQ_PROD, k)
        vc, vn, _ = tq.tq_encode(g, tq.TQ_MSE, v)
        with pytest.raises(tq.TQError):
            tq.tq_attend_decode(g, g, q, kc, kn, kg, vc, vn, 1, 64, None, None)
    k, v, q = _gqa_inputs(1, 1, 4, 64, 64, seed=3)
    g = tq.Quantizer(64, 3, 0)
    kc, kn, kg = tq.tq_encode(g, tq.TQ_PROD, k)
    vc, vn, _ = tq.tq_encode(g, tq.TQ_MSE, v)
    with pytest.raises(tq.TQError):
        tq.tq_attend_decode(g, g, q, kc, kn, kg, vc, vn, 1, 64, None, None, v_threshold=0.01)


def test_attend_custom_scale_and_same_quantizer():
    print("case: attend custom scale", flush=True)
    k, v, q = _gqa_inputs(1, 2, 8, 600, 128, seed=11)
    _run_case(k, v, q, 1, 2, 8, 600, 0, 3, scale=0.02, kseed=5, vseed=5)


def test_attend_one_round_chunks_ten_groups():
    """4-bit keys and values over 131072 tokens with 10 KV heads: the chunk
    kernel runs three workgroups per CU, 2048-token chunks would leave 640 of
    the 768 resident slots, and the chunking fills one round instead (at most
    76 chunks per group: 74 chunks of 1792 tokens).  The oracle checks two
    groups."""
    print("case: attend one-round chunks B=1 Hkv=10 Hq=40 N=131072 bits=4", flush=True)
    B, Hkv, Hq, N = 1, 10, 40, 131072
    k, v, q = _gqa_inputs(B, Hkv, Hq, N, 128, seed=77)
    w = _run_case(k, v, q, B, Hkv, Hq, N, 0, 4, groups=[(0, 0), (0, 9)])
    print("worst relative error", w)


@pytest.mark.parametrize("kbits,vbits", [(4, 2), (2, 4), (3, 1), (4, 3)])
def test_attend_asymmetric_bits(kbits, vbits):
    """Keys and values at different bit widths (each quantizer owns its own
    codebook); the chunk kernel is instantiated per (key bits, value bits)."""
    print(f"case: attend asymmetric K {kbits}-bit V {vbits}-bit", flush=True)
    k, v, q = _gqa_inputs(1, 4, 16, 2000, 128, seed=kbits * 10 + vbits)
    w = _run_case(k, v, q, 1, 4, 16, 1900, 100, kbits, vbits=vbits)
    print("worst relative error", w)


def test_attend_steep_logit_drop_within_chunk():
    """Regression: within each chunk the first 128-token step scores 122.5
    log2 units above the second (a weight ratio of 2^-122.5, still a normal
    float).  The accumulator rescale between the two steps must stay finite;
    the output is the oracle's attention to within the usual tolerance.  All
    keys share one direction u (fp32, so every key gets the same code and
    logit_t = n_t * L for the unit key's logit L, measured first).  Shape
    8 x 8 x 8192 gives chunks of two steps."""
    print("case: attend steep logit drop B=8 Hkv=8 Hq=32 N=8192", flush=True)
    B, Hkv, Hq, N, d = 8, 8, 32, 8192, 128
    rng = np.random.default_rng(21)
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    qt = torch.from_numpy(np.broadcast_to(u, (B, Hq, d)).astype(np.float32).copy()).to(_dev()).bfloat16()
    gk, _ = _pair(d, 3, 0)
    cu, nu, gu = tq.tq_encode(gk, tq.TQ_PROD, torch.from_numpy(u[None, None, :].astype(np.float32)).to(_dev()))
    L = float(tq.tq_scores(gk, qt[:1, :1].contiguous(), cu, nu, gu, 1, 1)[0, 0, 0]) / math.sqrt(d)
    assert L > 0.5 / math.sqrt(d)                        # <u, u> = 1 up to quantisation
    a_low = 7.0 / L                                      # scaled logit 7 nats
    a_high = a_low + 122.5 * math.log(2.0) / L           # 122.5 log2 units higher
    a = np.where((np.arange(N) % 256) < 128, a_high, a_low)
    k = (a[None, :, None] * u[None, None, :]).astype(np.float32)
    kt = torch.from_numpy(np.ascontiguousarray(np.broadcast_to(k, (B * Hkv, N, d)))).to(_dev())
    vt = torch.from_numpy(rng.standard_normal((B * Hkv, N, d)).astype(np.float32)).to(_dev()).bfloat16()
    w = _run_case(kt, vt, qt, B, Hkv, Hq, N, 0, 3, groups=[(0, 0), (7, 7)])
    print("worst relative error", w)


def _sparse_run(k, v, q, B, Hkv, Hq, n_comp, n_tail, bits, tau, groups=None):
    """tq_attend_decode_sparse against the oracle's dense attention: per
    element |gpu - oracle| <= 1e-3 max(|oracle_e|, ||oracle_row||/sqrt(d)) +
    the oracle's sparse-V bound (the largest change any allowed drop can make;
    drop set taken with a 1% margin on the threshold for the GPU's rounding
    of the weights).  Returns (worst excess ratio, dropped fraction of D)."""
    d = k.shape[-1]
    gk, ok = _pair(d, bits, 0)
    gv, ov = _pair(d, bits, 1)
    kcodes, kn, kg = tq.tq_encode(gk, tq.TQ_PROD, k[:, :n_comp].contiguous())
    vcodes, vn, _ = tq.tq_encode(gv, tq.TQ_MSE, v[:, :n_comp].contiguous())
    kt = k[:, n_comp:].contiguous().view(B, Hkv, n_tail, d) if n_tail else None
    vt = v[:, n_comp:].contiguous().view(B, Hkv, n_tail, d) if n_tail else None
    dense = tq.tq_attend_decode(gk, gv, q, kcodes, kn, kg, vcodes, vn, Hkv, n_comp, kt, vt).cpu().numpy()
    out = tq.tq_attend_decode(gk, gv, q, kcodes, kn, kg, vcodes, vn, Hkv, n_comp, kt, vt,
                              v_threshold=tau).cpu().numpy()
    G = Hq // Hkv
    kw, vw = P.to_u32(kcodes), P.to_u32(vcodes)
    kn, kg, vn = (t.cpu().numpy().astype(np.float64) for t in (kn, kg, vn))
    qs = q.float().cpu().numpy().astype(np.float64)
    kf, vf = k.float().cpu().numpy().astype(np.float64), v.float().cpu().numpy().astype(np.float64)
    perk, perv = gk.code_words(tq.TQ_PROD, 1, n_comp), gv.code_words(tq.TQ_MSE, 1, n_comp)
    worst, moved = 0.0, 0.0
    for (b, h) in (groups or [(b, h) for b in range(B) for h in range(Hkv)]):
        s = b * Hkv + h
        ki, kb = o.unpack_prod(kw[s * perk:(s + 1) * perk].reshape(n_comp, -1), bits - 1, d)
        vi = o.unpack_mse(vw[s * perv:(s + 1) * perv], n_comp, bits, d)
        sl = slice(s * n_comp, (s + 1) * n_comp)
        qq = qs[b, h * G:(h + 1) * G]
        tails = (kf[s, n_comp:], vf[s, n_comp:]) if n_tail else (None, None)
        ref = o.attend(ok, ov, qq, ki, kb, kn[sl], kg[sl], vi, vn[sl], *tails)
        bound = o.sparse_v_bound(ok, ov, qq, ki, kb, kn[sl], kg[sl], vi, vn[sl], tau, *tails, margin=1.01)
        floor = np.linalg.norm(ref, axis=1, keepdims=True) / math.sqrt(d)
        tol = 1e-3 * np.maximum(np.abs(ref), floor) + bound
        err = np.abs(out[b, h * G:(h + 1) * G] - ref)
        assert np.all(err <= tol + 1e-30), f"sparse V error beyond the bound ({np.max(err / tol):.3g})"
        worst = max(worst, float(np.max(err / tol)))
        moved = max(moved, float(np.max(np.abs(out[b, h * G:(h + 1) * G] - dense[b, h * G:(h + 1) * G]))))
    return worst, moved


@pytest.mark.parametrize("B,Hkv,Hq,N,tail,bits", [(2, 2, 8, 1000, 0, 3), (1, 2, 8, 777, 37, 4), (2, 8, 32, 4096, 0, 3)])
def test_attend_sparse_zero_threshold_is_dense(B, Hkv, Hq, N, tail, bits):
    """v_threshold = 0 reproduces tq_attend_decode bit for bit."""
    print(f"case: attend sparse tau=0 B={B} Hkv={Hkv} Hq={Hq} N={N} tail={tail} bits={bits}", flush=True)
    k, v, q = _gqa_inputs(B, Hkv, Hq, N, 128, seed=N + 5)
    gk, _ = _pair(128, bits, 0)
    gv, _ = _pair(128, bits, 1)
    kc, kn, kg = tq.tq_encode(gk, tq.TQ_PROD, k[:, :N - tail].contiguous())
    vc, vn, _ = tq.tq_encode(gv, tq.TQ_MSE, v[:, :N - tail].contiguous())
    kt = k[:, N - tail:].contiguous().view(B, Hkv, tail, 128) if tail else None
    vt = v[:, N - tail:].contiguous().view(B, Hkv, tail, 128) if tail else None
    a = tq.tq_attend_decode(gk, gv, q, kc, kn, kg, vc, vn, Hkv, N - tail, kt, vt)
    b = tq.tq_attend_decode(gk, gv, q, kc, kn, kg, vc, vn, Hkv, N - tail, kt, vt, v_threshold=0.0)
    assert torch.equal(a, b)


@pytest.mark.parametrize("B,Hkv,Hq,N,tail,bits,tau,qscale", [
    (2, 2, 8, 1000, 0, 3, 1e-4, 1.0), (1, 2, 8, 777, 37, 4, 1e-2, 1.0), (2, 8, 32, 4096, 0, 3, 0.3, 3.0),
    (1, 4, 16, 3000, 100, 3, 1e-3, 3.0), (1, 1, 4, 129, 0, 2, 0.9, 1.0)])
def test_attend_sparse_within_bound(B, Hkv, Hq, N, tail, bits, tau, qscale):
    """Sparse V against the oracle's dense attention plus the drop bound;
    qscale 3 makes the softmax peaked (logits / sqrt(d) with std about 9) so
    that whole 128-token steps drop out and skip their value MFMAs."""
    print(f"case: attend sparse tau={tau} B={B} Hkv={Hkv} Hq={Hq} N={N} tail={tail} bits={bits} qscale={qscale}",
          flush=True)
    k, v, q = _gqa_inputs(B, Hkv, Hq, N, 128, seed=N + 11)
    q = (q.float() * qscale).bfloat16()
    worst, moved = _sparse_run(k, v, q, B, Hkv, Hq, N - tail, tail, bits, tau, groups=[(0, 0), (B - 1, Hkv - 1)])
    print("worst error / tolerance", worst, "largest change from dense", moved)


def test_attend_sparse_full_size_gqa():
    """The GQA decode layer at full size with v_threshold 1e-3."""
    print("case: attend sparse full size gqa tau=1e-3", flush=True)
    wl = W.gqa_layer()
    B, Hkv, Hq, N = wl.meta["B"], wl.meta["Hkv"], wl.meta["Hq"], wl.meta["N"]
    k = _bf16(wl.arrays["k_bf16"]).view(B * Hkv, N, 128)
    v = _bf16(wl.arrays["v_bf16"]).view(B * Hkv, N, 128)
    q = _bf16(wl.arrays["q_bf16"])
    worst, moved = _sparse_run(k, v, q, B, Hkv, Hq, N, 0, wl.bits, 1e-3, groups=[(0, 0), (B - 1, Hkv - 1)])
    print("worst error / tolerance", worst, "largest change from dense", moved)


def test_attend_sparse_rejects_bad_threshold():
    k, v, q = _gqa_inputs(1, 1, 4, 64, 128, seed=3)
    gk, _ = _pair(128, 3, 0)
    gv, _ = _pair(128, 3, 1)
    kc, kn, kg = tq.tq_encode(gk, tq.TQ_PROD, k.contiguous())
    vc, vn, _ = tq.tq_encode(gv, tq.TQ_MSE, v.contiguous())
    for bad in (-0.1, 1.0, float("nan")):
        with pytest.raises(RuntimeError):
            tq.tq_attend_decode(gk, gv, q, kc, kn, kg, vc, vn, 1, 64, v_threshold=bad)
