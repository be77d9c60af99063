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


def test_attend_custom_scale_and_same_quantizer():
    print("case: attend custom scale", flush=True)
    k, v, q = _gqa_inputs(1, 2, 8, 600, 128, seed=11)
    _run_case(k, v, q, 1, 2, 8, 600, 0, 3, scale=0.02, kseed=5, vseed=5)


@pytest.mark.parametrize("name", ["gqa", "long"])
def test_attend_full_size_sampled(name):
    """The GQA decode layer and long-context workloads at full size; the
    oracle checks the outputs of a few (batch, KV head) groups."""
    print(f"case: attend full size {name}", flush=True)
    wl = W.gqa_layer() if name == "gqa" else W.long_context()
    B, Hkv, Hq, N = wl.meta["B"], wl.meta["Hkv"], wl.meta["Hq"], wl.meta["N"]
    tail = wl.meta.get("tail", 0)
    k = _bf16(wl.arrays["k_bf16"]).view(B * Hkv, N, 128)
    v = _bf16(wl.arrays["v_bf16"]).view(B * Hkv, N, 128)
    q = _bf16(wl.arrays["q_bf16"])
    groups = [(0, 0), (B - 1, Hkv - 1)]
    w = _run_case(k, v, q, B, Hkv, Hq, N - tail, tail, wl.bits, groups=groups, kseed=0, vseed=0)
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
