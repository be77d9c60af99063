"""GPU parity: tq_encode / tq_decode / tq_scores through the C ABI against the
CPU oracle on the same seeded inputs (see tests/parity.py for tolerances)."""
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


_QZ = {}


def _pair(d, bits, seed=0):
    key = (d, bits, seed)
    if key not in _QZ:
        _QZ[key] = (tq.Quantizer(d, bits, seed), o.Quantizer(d, bits, seed))
    return _QZ[key]


def _up(a, bf16=False):
    t = torch.from_numpy(np.ascontiguousarray(a)).to(_dev())
    return t.to(torch.bfloat16) if bf16 else t


def _encode_prod(g, x, bf16):
    xt = _up(x.astype(np.float32), bf16)
    codes, norms, gam = tq.tq_encode(g, tq.TQ_PROD, xt)
    torch.cuda.synchronize()
    xs = xt.float().cpu().numpy().astype(np.float64).reshape(-1, x.shape[-1])
    N = xs.shape[0]
    return xs, P.to_u32(codes)[: g.code_words(tq.TQ_PROD, 1, N)], norms.cpu().numpy()[:N], gam.cpu().numpy()[:N]


def test_encode_tiny_workload():
    wl = W.tiny()
    g, oq = _pair(128, 3)
    print("case: tiny workload 4096x128 fp32 bits=3", flush=True)
    xs, codes, norms, gam = _encode_prod(g, wl.arrays["x"], False)
    _, _, st = P.check_prod_codes(oq, xs, codes, norms, gam)
    print(st)


@pytest.mark.parametrize("d,bits,nseq,n,bf16", [
    (128, 2, 3, 1000, True), (128, 4, 2, 777, True), (128, 3, 1, 64, False), (128, 3, 2, 1, False),
    (200, 2, 1, 3000, False), (200, 4, 1, 1500, False), (16, 3, 2, 100, False), (48, 2, 1, 65, False),
    (3, 2, 1, 10, False), (256, 3, 1, 130, True),
    (201, 3, 2, 333, False)])   # d > 128 and not a multiple of 4: the element-wise tile load
def test_encode_prod_shapes(d, bits, nseq, n, bf16):
    print(f"case: prod d={d} bits={bits} nseq={nseq} n={n} bf16={bf16}", flush=True)
    rng = np.random.default_rng(d * 100 + bits)
    x = (rng.standard_normal((nseq, n, d)) * np.exp(rng.uniform(0, math.log(50), (1, 1, d)))).astype(np.float32)
    g, oq = _pair(d, bits)
    xs, codes, norms, gam = _encode_prod(g, x, bf16)
    P.check_prod_codes(oq, xs, codes, norms, gam)


@pytest.mark.parametrize("d,bits,nseq,n,bf16", [
    (128, 3, 4, 1000, True), (128, 4, 2, 4101, True), (16, 1, 1, 33, False), (128, 2, 3, 64, False),
    (200, 4, 1, 70, False), (130, 2, 1, 200, False)])
def test_encode_mse_shapes(d, bits, nseq, n, bf16):
    print(f"case: mse d={d} bits={bits} nseq={nseq} n={n} bf16={bf16}", flush=True)
    rng = np.random.default_rng(d + bits)
    x = rng.standard_normal((nseq, n, d)).astype(np.float32)
    g, oq = _pair(d, bits)
    xt = _up(x, bf16)
    codes, norms, _ = tq.tq_encode(g, tq.TQ_MSE, xt)
    torch.cuda.synchronize()
    xs = xt.float().cpu().numpy().astype(np.float64)
    cw = P.to_u32(codes)
    per = g.code_words(tq.TQ_MSE, 1, n)
    nn = norms.cpu().numpy()
    for s in range(nseq):
        P.check_mse_codes(oq, xs[s], cw[s * per:(s + 1) * per], nn[s * n:(s + 1) * n])


@pytest.mark.parametrize("bits,nseq,n,bf16", [
    (2, 3, 40001, False), (3, 2, 33000, True), (4, 2, 40033, False), (4, 3, 21000, True)])
def test_encode_prod_d128_many_tiles_per_workgroup(bits, nseq, n, bf16):
    """d = 128 prod keys over hundreds of tiles, so every workgroup of the
    persistent grid runs its pipeline (load, rotation, projection, store)
    through several tiles; zero rows at tile edges and a ragged tail."""
    print(f"case: prod d=128 bits={bits} nseq={nseq} n={n} bf16={bf16} (many tiles)", flush=True)
    rng = np.random.default_rng(7000 + bits)
    x = (rng.standard_normal((nseq, n, 128)) * np.exp(rng.uniform(0, math.log(50), (1, 1, 128)))).astype(np.float32)
    for r in (0, 63, 64, 4095, n - 1):
        x[nseq - 1, r] = 0.0
    g, oq = _pair(128, bits)
    xs, codes, norms, gam = _encode_prod(g, x, bf16)
    P.check_prod_codes(oq, xs, codes, norms, gam)
    zero = (nseq - 1) * n + np.array([0, 63, 64, 4095, n - 1])
    assert np.all(norms[zero] == 0) and np.all(gam[zero] == 0)


def test_encode_zero_vectors_and_empty():
    print("case: zero vectors", flush=True)
    g, oq = _pair(128, 3)
    x = np.zeros((5, 128), dtype=np.float32)
    x[2] = 1.0
    xs, codes, norms, gam = _encode_prod(g, x, False)
    idx, bits, _ = P.check_prod_codes(oq, xs, codes, norms, gam)
    assert np.all(idx[0] == 1) and np.all(bits[0] == 1) and norms[0] == 0 and gam[0] == 0
    # n = 0 is a no-op
    e = torch.empty((0, 128), device=_dev())
    tq.tq_encode(g, tq.TQ_PROD, e)
    torch.cuda.synchronize()


@pytest.mark.parametrize("mode,d,bits,n", [(0, 128, 3, 300), (0, 200, 4, 50), (1, 128, 4, 100), (0, 16, 2, 40)])
def test_decode_matches_oracle(mode, d, bits, n):
    print(f"case: decode mode={mode} d={d} bits={bits}", flush=True)
    rng = np.random.default_rng(7)
    x = rng.standard_normal((n, d)).astype(np.float32) * 3
    g, oq = _pair(d, bits)
    xt = _up(x)
    codes, norms, gam = tq.tq_encode(g, mode, xt)
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
    assert err.max() < 1e-5


def _scores_case(d, bits, B, Hkv, Hq, n, bf16, seed=0):
    rng = np.random.default_rng(seed)
    g, oq = _pair(d, bits)
    k = (rng.standard_normal((B * Hkv, n, d)) * np.exp(rng.uniform(0, math.log(50), (B * Hkv, 1, d)))).astype(np.float32)
    q = rng.standard_normal((B, Hq, d)).astype(np.float32)
    kt = _up(k, bf16)
    qt = _up(q, bf16)
    codes, norms, gam = tq.tq_encode(g, tq.TQ_PROD, kt)
    logits = tq.tq_scores(g, qt, codes, norms, gam, Hkv, n).cpu().numpy()
    cw = P.to_u32(codes)
    nn = norms.cpu().numpy().astype(np.float64)
    gg = gam.cpu().numpy().astype(np.float64)
    qs = qt.float().cpu().numpy().astype(np.float64)
    G = Hq // Hkv
    per = g.code_words(tq.TQ_PROD, 1, n)
    worst = 0.0
    for b in range(B):
        for h in range(Hkv):
            s = b * Hkv + h
            idx, bits01 = o.unpack_prod(cw[s * per:(s + 1) * per].reshape(n, -1), bits - 1, d)
            qq = qs[b, h * G:(h + 1) * G]
            ref = o.scores(oq, qq, idx, bits01, nn[s * n:(s + 1) * n], gg[s * n:(s + 1) * n])
            worst = max(worst, P.check_logits(logits[b, h * G:(h + 1) * G], ref, np.linalg.norm(qq, axis=1),
                                              nn[s * n:(s + 1) * n], d))
    return worst


def test_scores_tiny_workload():
    print("case: scores tiny workload 16 x 4096", flush=True)
    wl = W.tiny()
    g, oq = _pair(128, 3)
    xt = _up(wl.arrays["x"])
    qt = _up(wl.arrays["q"][None])
    codes, norms, gam = tq.tq_encode(g, tq.TQ_PROD, xt)
    logits = tq.tq_scores(g, qt, codes, norms, gam, 1, 4096)[0].cpu().numpy()
    idx, bits01 = o.unpack_prod(P.to_u32(codes).reshape(4096, -1), 2, 128)
    nn = norms.cpu().numpy().astype(np.float64)
    ref = o.scores(oq, wl.arrays["q"].astype(np.float64), idx, bits01, nn, gam.cpu().numpy().astype(np.float64))
    w = P.check_logits(logits, ref, np.linalg.norm(wl.arrays["q"], axis=1).astype(np.float64), nn, 128)
    print("worst relative logit error", w)


@pytest.mark.parametrize("d,bits,B,Hkv,Hq,n,bf16", [
    (128, 3, 2, 2, 8, 777, True), (128, 2, 1, 4, 4, 1000, True), (128, 4, 1, 2, 8, 513, True),
    (128, 3, 1, 1, 5, 300, False), (200, 2, 1, 1, 6, 700, False), (200, 4, 1, 2, 2, 333, False),
    (16, 3, 1, 1, 4, 50, False), (48, 2, 2, 1, 2, 17, False)])
def test_scores_shapes(d, bits, B, Hkv, Hq, n, bf16):
    print(f"case: scores d={d} bits={bits} B={B} Hkv={Hkv} Hq={Hq} n={n}", flush=True)
    w = _scores_case(d, bits, B, Hkv, Hq, n, bf16)
    print("worst relative logit error", w)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_decode_layer_full_size_sampled(bits):
    """Single-layer decode workload at full size (32 heads x 8192 keys):
    every key is encoded on the GPU and checked against the oracle (head by
    head), and all 32 x 8192 logits are checked on identical codes."""
    print(f"case: decode layer full size bits={bits}", flush=True)
    wl = W.decode_layer(bits)
    g, oq = _pair(128, bits)
    kt = torch.from_numpy(wl.arrays["k_bf16"].view(np.int16)).to(_dev()).view(torch.bfloat16)
    qt = torch.from_numpy(wl.arrays["q_bf16"].view(np.int16)).to(_dev()).view(torch.bfloat16)[None]
    codes, norms, gam = tq.tq_encode(g, tq.TQ_PROD, kt)
    logits = tq.tq_scores(g, qt, codes, norms, gam, 32, 8192)[0].cpu().numpy()
    cw = P.to_u32(codes).reshape(32 * 8192, -1)
    nn = norms.cpu().numpy().astype(np.float64)
    gg = gam.cpu().numpy().astype(np.float64)
    kv = wl.arrays["k"].reshape(-1, 128).astype(np.float64)
    qv = wl.arrays["q"].astype(np.float64)
    for h in range(32):
        sl = slice(h * 8192, (h + 1) * 8192)
        P.check_prod_codes(oq, kv[sl], cw[sl].reshape(-1), nn[sl], gg[sl])
        idx, bits01 = o.unpack_prod(cw[sl].reshape(-1).reshape(8192, -1), bits - 1, 128)
        ref = o.scores(oq, qv[h:h + 1], idx, bits01, nn[sl], gg[sl])
        P.check_logits(logits[h:h + 1], ref, np.linalg.norm(qv[h:h + 1], axis=1), nn[sl], 128)


def test_binding_rejects_mis_sized_buffers():
    """The C ABI takes no buffer lengths, so the binding checks every tensor
    it forwards (shape, dtype, element count) and raises before any launch."""
    print("case: binding argument checks", flush=True)
    g, _ = _pair(128, 3)
    dev = _dev()
    x = torch.randn(2, 100, 128, device=dev)
    codes, norms, gam = tq.tq_encode(g, tq.TQ_PROD, x)
    q = torch.randn(1, 4, 128, device=dev)
    with pytest.raises(ValueError):                       # 4-D input
        tq.tq_encode(g, tq.TQ_PROD, x[None])
    with pytest.raises(ValueError):                       # codes too short
        tq.tq_encode(g, tq.TQ_PROD, x, out=(codes[:10], norms, gam))
    with pytest.raises(ValueError):                       # norms too short
        tq.tq_encode(g, tq.TQ_PROD, x, out=(codes, norms[:199], gam))
    with pytest.raises(TypeError):                        # wrong dtype
        tq.tq_encode(g, tq.TQ_PROD, x, out=(codes, norms.double(), gam))
    with pytest.raises(ValueError):                       # query d differs from the quantizer's
        tq.tq_scores(g, torch.randn(1, 4, 64, device=dev), codes, norms, gam, 2, 100)
    with pytest.raises(ValueError):                       # more keys than the codes hold
        tq.tq_scores(g, q, codes, norms, gam, 1, 201)
    with pytest.raises(ValueError):                       # output too small
        tq.tq_scores(g, q, codes, norms, gam, 1, 200, out=torch.empty(4, 100, device=dev))
    with pytest.raises(ValueError):                       # workspace too small
        tq.tq_scores(g, q, codes, norms, gam, 1, 200, workspace=torch.empty(16, dtype=torch.uint8, device=dev))
    with pytest.raises(ValueError):                       # decode output too small
        tq.tq_decode(g, tq.TQ_PROD, codes, norms, gam, 2, 100, out=torch.empty(2, 99, 128, device=dev))
    gv = tq.Quantizer(128, 3, 1)
    vc, vn, _ = tq.tq_encode(gv, tq.TQ_MSE, x)
    qa = torch.randn(2, 4, 128, device=dev)
    with pytest.raises(ValueError):                       # tail of the wrong shape
        tq.tq_attend_decode(g, gv, qa, codes, norms, gam, vc, vn, 1, 100,
                            torch.zeros(2, 1, 5, 128, device=dev, dtype=torch.bfloat16),
                            torch.zeros(2, 1, 6, 128, device=dev, dtype=torch.bfloat16))
    with pytest.raises(ValueError):                       # value codes too short
        tq.tq_attend_decode(g, gv, qa, codes, norms, gam, vc[:50], vn, 1, 100)
    # the correct call still runs
    out = tq.tq_attend_decode(g, gv, qa, codes, norms, gam, vc, vn, 1, 100)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
