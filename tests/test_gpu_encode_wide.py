"""GPU parity of the eight-wave encoder (128 < d <= 256, rows in 16-byte
runs): prod keys, values and MSE-only keys against the oracle on shapes with
more tiles than resident workgroups, so every workgroup encodes several
64-vector tiles through its double buffers, and a sampled check of a large
d = 200 float database (the vector-search dimension)."""
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


def _pair(d, bits, seed=0, rotation=tq.TQ_ROT_HAAR):
    key = (d, bits, seed, rotation)
    if key not in _QZ:
        _QZ[key] = (tq.Quantizer(d, bits, seed, rotation),
                    o.Quantizer(d, bits, seed, rotation_kind="hadamard" if rotation == tq.TQ_ROT_HADAMARD else "haar"))
    return _QZ[key]


def _data(rng, nseq, n, d):
    # per-channel scales log-uniform over [1, 50] (anisotropic keys, as the decode-layer workload)
    return (rng.standard_normal((nseq, n, d)) * np.exp(rng.uniform(0, math.log(50), (nseq, 1, d)))).astype(np.float32)


def _check(g, oq, mode, xt, nseq, n, rows=None):
    m = {"prod": tq.TQ_PROD, "mse": tq.TQ_MSE, "mse_keys": tq.TQ_MSE_KEYS}[mode]
    codes, norms, gam = tq.tq_encode(g, m, xt)
    torch.cuda.synchronize()
    xs = xt.float().cpu().numpy().astype(np.float64)
    cw = P.to_u32(codes)
    per = g.code_words(m, 1, n)
    nn = norms.cpu().numpy()
    gg = gam.cpu().numpy() if gam is not None else None
    d = xs.shape[-1]
    for s in range(nseq):
        sl = slice(s * n, (s + 1) * n)
        c = cw[s * per:(s + 1) * per]
        if mode == "prod":
            if rows is None:
                P.check_prod_codes(oq, xs[s], c, nn[sl], gg[sl])
            else:
                words = c.reshape(n, -1)[rows]
                P.check_prod_codes(oq, xs[s][rows], words.reshape(-1), nn[sl][rows], gg[sl][rows])
        elif mode == "mse":
            P.check_mse_codes(oq, xs[s], c, nn[sl])
        else:
            if rows is None:
                P.check_mse_key_codes(oq, xs[s], c, nn[sl])
            else:
                words = c.reshape(n, -1)[rows]
                P.check_mse_key_codes(oq, xs[s][rows], words.reshape(-1), nn[sl][rows])


@pytest.mark.parametrize("d,bits,mode,nseq,n,bf16", [
    (256, 3, "prod", 4, 8200, True), (256, 4, "prod", 2, 8000, False), (200, 4, "prod", 4, 4133, False),
    (160, 2, "prod", 4, 8197, True), (224, 3, "prod", 2, 9001, False),
    (256, 3, "mse", 8, 8192, True), (200, 4, "mse", 4, 8227, False), (192, 2, "mse", 6, 4100, True),
    (256, 4, "mse_keys", 4, 8200, False), (208, 3, "mse_keys", 4, 4099, True),
    (256, 3, "prod", 1, 1, True), (200, 2, "mse", 1, 33, False)])
def test_wide_encoder_multi_tile(d, bits, mode, nseq, n, bf16):
    """Every code of every sequence, ragged tails, both input types, d from
    160 to 256 (partial last group where d is not a multiple of 32)."""
    print(f"case: wide encoder d={d} bits={bits} {mode} nseq={nseq} n={n} bf16={bf16}", flush=True)
    g, oq = _pair(d, bits)
    if mode == "mse_keys":
        g, oq = _pair(d, bits, seed=1)
    x = _data(np.random.default_rng(d * 100 + bits * 10 + n), nseq, n, d)
    x[:, 0] = 0.0   # a zero vector in every sequence
    xt = torch.from_numpy(x).to(_dev())
    if bf16:
        xt = xt.bfloat16()
    _check(g, oq, mode, xt, nseq, n)


def test_wide_encoder_hadamard_prod_keys():
    """Prod keys under the Hadamard rotation at d = 256 take the eight-wave
    kernel with the +-1 matrix as a general one."""
    print("case: wide encoder hadamard prod d=256 bits=3 nseq=4 n=5000", flush=True)
    g, oq = _pair(256, 3, rotation=tq.TQ_ROT_HADAMARD)
    x = _data(np.random.default_rng(77), 4, 5000, 256)
    _check(g, oq, "prod", torch.from_numpy(x).to(_dev()).bfloat16(), 4, 5000)


def test_wide_encoder_vector_search_database_sampled():
    """262144 x 200 float vectors of the vector-search law (4096 tiles, about
    16 per persistent workgroup at one per CU): 4-bit prod codes of every 61st
    row, which visits every position in a tile and every workgroup."""
    print("case: wide encoder 262144 x 200 fp32 4-bit prod, sampled", flush=True)
    wl = W.vector_search(4, n=262144, nq=16)
    x = wl.arrays["x"].astype(np.float32)
    n = x.shape[0]
    g, oq = _pair(200, 4)
    rows = np.arange(0, n, 61)
    _check(g, oq, "prod", torch.from_numpy(x).to(_dev()).view(1, n, 200), 1, n, rows=rows)
