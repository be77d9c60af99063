"""GPU parity at full size, on the kernel paths the benchmark times.

The GQA decode layer (batch 8, 8 KV heads, 32 query heads, 32768 tokens,
d = 128, 3-bit prod keys and 3-bit values) and the long-context layer
(131072 tokens, the last 256 kept bf16, 4-bit) are encoded, scored and
attended on the GPU with the same calls and launch shapes as the benchmark:
one tq_encode over all sequences (persistent encoder workgroups that loop
over many tiles), tq_query_prep + tq_scores_from_prep (several 64-key
batches per scan wave through the LDS ring), and tq_attend_decode.  Then:

  * every key code and every value code of every sequence is checked against
    the oracle's encoding (tests/parity.py: bit-exact up to the decision
    band, at most 1e-4 of coordinates flipped, norms and gammas to 1e-5);
  * every logit of every (batch, KV head) group is checked against the
    oracle's logits on the GPU's codes (relative 1e-3 with the floor
    ||q|| n / sqrt(d));
  * the attention output of every group is checked against the oracle's
    attention on the GPU's codes.

The ragged cases at the end run the scan with several batches per wave and
n not a multiple of 4 (element-wise logit stores), and the value encoder
with more tiles than workgroups and a partial last 32-token block.
"""
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


def _bf16(u16):
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).to(_dev()).view(torch.bfloat16)


def _scan_batches_per_wave(groups, n):
    """Batches of 64 keys the busiest scan wave takes (the launch rule of the
    logits kernel: about 4096 waves over all groups)."""
    nbatch = -(-n // 64)
    bx = max(1, min(-(-1024 // groups), -(-nbatch // 4)))
    return -(-nbatch // (4 * bx))


def _run_layer(wl, n_tail, bits=None, vbits=None):
    """Encode, score and attend a GQA-shaped workload the way the benchmark
    does (keys at `bits`, values at `vbits`, both the workload's by default);
    return every GPU output and the float inputs as numpy arrays."""
    B, Hkv, Hq, N, d = wl.meta["B"], wl.meta["Hkv"], wl.meta["Hq"], wl.meta["N"], wl.d
    bits = bits or wl.bits
    vbits = vbits or bits
    n_comp = N - n_tail
    nseq = B * Hkv
    qz = tq.Quantizer(d, bits, 0)
    qv = qz if vbits == bits else tq.Quantizer(d, vbits, 0)
    k_all = _bf16(wl.arrays["k_bf16"]).view(nseq, N, d)
    v_all = _bf16(wl.arrays["v_bf16"]).view(nseq, N, d)
    q = _bf16(wl.arrays["q_bf16"])
    k = k_all[:, :n_comp].contiguous()
    v = v_all[:, :n_comp].contiguous()
    kt = k_all[:, n_comp:].contiguous().view(B, Hkv, n_tail, d) if n_tail else None
    vt = v_all[:, n_comp:].contiguous().view(B, Hkv, n_tail, d) if n_tail else None
    kc, kn, kg = tq.tq_encode(qz, tq.TQ_PROD, k)
    vc, vn, _ = tq.tq_encode(qv, tq.TQ_MSE, v)
    ws = tq.tq_query_prep(qz, q, Hkv)
    logits = tq.tq_scores_from_prep(qz, B, Hq, Hkv, kc, kn, kg, n_comp, ws)
    logits_call = tq.tq_scores(qz, q, kc, kn, kg, Hkv, n_comp)
    out = tq.tq_attend_decode(qz, qv, q, kc, kn, kg, vc, vn, Hkv, n_comp, kt, vt)
    torch.cuda.synchronize()
    assert torch.equal(logits, logits_call), "tq_scores and query prep + scan differ"
    del logits_call, k, v, k_all, v_all
    return {
        "B": B, "Hkv": Hkv, "Hq": Hq, "N": N, "n_comp": n_comp, "n_tail": n_tail, "d": d, "bits": bits,
        "kw": P.to_u32(kc).reshape(nseq, n_comp, -1), "kn": kn.cpu().numpy().reshape(nseq, n_comp),
        "kg": kg.cpu().numpy().reshape(nseq, n_comp),
        "vw": P.to_u32(vc).reshape(nseq, -1), "vn": vn.cpu().numpy().reshape(nseq, n_comp),
        "logits": logits.cpu().numpy(), "out": out.cpu().numpy(),
        "k": wl.arrays["k"].reshape(nseq, N, d), "v": wl.arrays["v"].reshape(nseq, N, d),
        "q": wl.arrays["q"], "oq": o.Quantizer(d, bits, 0), "ov": o.Quantizer(d, vbits, 0), "vbits": vbits,
    }


@pytest.fixture(scope="module")
def gqa():
    print("case: full-size GQA layer B=8 Hkv=8 Hq=32 N=32768 d=128 3-bit (encode, scan, attend)", flush=True)
    r = _run_layer(W.gqa_layer(), 0)
    print("scan batches per wave:", _scan_batches_per_wave(r["B"] * r["Hkv"], r["n_comp"]), flush=True)
    return r


@pytest.fixture(scope="module")
def long_ctx():
    print("case: full-size long context B=1 Hkv=8 Hq=32 N=131072 tail=256 d=128 4-bit (encode, scan, attend)",
          flush=True)
    r = _run_layer(W.long_context(), 256)
    print("scan batches per wave:", _scan_batches_per_wave(r["B"] * r["Hkv"], r["n_comp"]), flush=True)
    return r


def _check_key_codes(r, seqs):
    flips = 0
    for s in seqs:
        x = r["k"][s, :r["n_comp"]].astype(np.float64)
        _, _, st = P.check_prod_codes(r["oq"], x, r["kw"][s].reshape(-1), r["kn"][s], r["kg"][s])
        flips += st["index_flips"] + st["bit_flips"]
    return flips


def _check_value_codes(r, seqs):
    flips = 0
    for s in seqs:
        x = r["v"][s, :r["n_comp"]].astype(np.float64)
        _, st = P.check_mse_codes(r["ov"], x, r["vw"][s], r["vn"][s])
        flips += st["index_flips"]
    return flips


def _check_logits(r):
    d, bits, n = r["d"], r["bits"], r["n_comp"]
    G = r["Hq"] // r["Hkv"]
    worst = 0.0
    for b in range(r["B"]):
        for h in range(r["Hkv"]):
            s = b * r["Hkv"] + h
            idx, b01 = o.unpack_prod(r["kw"][s], bits - 1, d)
            qq = r["q"][b, h * G:(h + 1) * G].astype(np.float64)
            nn = r["kn"][s].astype(np.float64)
            ref = o.scores(r["oq"], qq, idx, b01, nn, r["kg"][s].astype(np.float64))
            worst = max(worst, P.check_logits(r["logits"][b, h * G:(h + 1) * G], ref, np.linalg.norm(qq, axis=1),
                                              nn, d))
    return worst


def _check_attention(r):
    d, bits, n = r["d"], r["bits"], r["n_comp"]
    G = r["Hq"] // r["Hkv"]
    worst = 0.0
    for b in range(r["B"]):
        for h in range(r["Hkv"]):
            s = b * r["Hkv"] + h
            ki, kb = o.unpack_prod(r["kw"][s], bits - 1, d)
            vi = o.unpack_mse(r["vw"][s], n, r["vbits"], d)
            tail_k = r["k"][s, n:].astype(np.float64) if r["n_tail"] else None
            tail_v = r["v"][s, n:].astype(np.float64) if r["n_tail"] else None
            ref = o.attend(r["oq"], r["ov"], r["q"][b, h * G:(h + 1) * G].astype(np.float64), ki, kb,
                           r["kn"][s].astype(np.float64), r["kg"][s].astype(np.float64), vi,
                           r["vn"][s].astype(np.float64), tail_k, tail_v)
            worst = max(worst, P.check_attention(r["out"][b, h * G:(h + 1) * G], ref))
    return worst


@pytest.mark.parametrize("half", [0, 1])
def test_gqa_key_codes_every_sequence(gqa, half):
    seqs = range(32 * half, 32 * half + 32)
    print("key code flips:", _check_key_codes(gqa, seqs))


@pytest.mark.parametrize("half", [0, 1])
def test_gqa_value_codes_every_sequence(gqa, half):
    seqs = range(32 * half, 32 * half + 32)
    print("value code flips:", _check_value_codes(gqa, seqs))


def test_gqa_logits_every_group(gqa):
    assert _scan_batches_per_wave(64, 32768) == 8
    print("worst relative logit error", _check_logits(gqa))


def test_gqa_attention_every_group(gqa):
    print("worst relative attention error", _check_attention(gqa))


def test_long_key_codes_every_sequence(long_ctx):
    print("key code flips:", _check_key_codes(long_ctx, range(8)))


def test_long_value_codes_every_sequence(long_ctx):
    print("value code flips:", _check_value_codes(long_ctx, range(8)))


def test_long_logits_every_group(long_ctx):
    assert _scan_batches_per_wave(8, 130816) == 4
    print("worst relative logit error", _check_logits(long_ctx))


def test_long_attention_every_group(long_ctx):
    print("worst relative attention error", _check_attention(long_ctx))


@pytest.mark.parametrize("width", [3.5, 2.5])
def test_gqa_fractional_width_every_group(width):
    """The GQA layer at a fractional cache width (the mean over key and value
    coordinates): 3.5 bits = 4-bit prod keys (3-bit index + QJL) with 3-bit
    values, 2.5 bits = 3-bit keys with 2-bit values.  Every logit and every
    group's attention output checked; key and value codes of 8 sequences
    (every 8th, so every batch) checked."""
    bits, vbits = o.kv_width_config(width)
    print(f"case: full-size GQA layer at {width} bits (keys {bits}, values {vbits})", flush=True)
    r = _run_layer(W.gqa_layer(), 0, bits, vbits)
    print("key code flips:", _check_key_codes(r, range(0, 64, 8)))
    print("value code flips:", _check_value_codes(r, range(0, 64, 8)))
    print("worst relative logit error", _check_logits(r))
    print("worst relative attention error", _check_attention(r))


@pytest.mark.parametrize("B,Hkv,Hq,n,bits", [(4, 8, 32, 32767, 3), (1, 4, 24, 100003, 4), (2, 2, 2, 262143, 2)])
def test_scores_ragged_multi_batch(B, Hkv, Hq, n, bits):
    """The scan with several 64-key batches per wave (the ring refill) and n
    not a multiple of 4 (element-wise logit stores); G = 6 leaves the second
    row tile half empty.  Every code and every logit is checked."""
    G = Hq // Hkv
    groups = B * Hkv * -(-G // 4)
    print(f"case: scores ragged B={B} Hkv={Hkv} Hq={Hq} n={n} bits={bits} "
          f"batches/wave={_scan_batches_per_wave(groups, n)}", flush=True)
    assert _scan_batches_per_wave(groups, n) > 1
    rng = np.random.default_rng(n + bits)
    d = 128
    k = (rng.standard_normal((B * Hkv, n, d), dtype=np.float32)
         * np.exp(rng.uniform(0, math.log(50), (B * Hkv, 1, d))).astype(np.float32))
    q = rng.standard_normal((B, Hq, d), dtype=np.float32)
    g = tq.Quantizer(d, bits, 0)
    oq = o.Quantizer(d, bits, 0)
    kt = torch.from_numpy(k).to(_dev()).bfloat16()
    qt = torch.from_numpy(q).to(_dev())
    codes, norms, gam = tq.tq_encode(g, tq.TQ_PROD, kt)
    logits = tq.tq_scores(g, qt, codes, norms, gam, Hkv, n).cpu().numpy()
    kw = P.to_u32(codes).reshape(B * Hkv, n, -1)
    nn = norms.cpu().numpy().reshape(B * Hkv, n).astype(np.float64)
    gg = gam.cpu().numpy().reshape(B * Hkv, n).astype(np.float64)
    ks = kt.float().cpu().numpy().astype(np.float64)
    worst = 0.0
    for b in range(B):
        for h in range(Hkv):
            s = b * Hkv + h
            P.check_prod_codes(oq, ks[s], kw[s].reshape(-1), nn[s].astype(np.float32), gg[s].astype(np.float32))
            idx, b01 = o.unpack_prod(kw[s], bits - 1, d)
            qq = q[b, h * G:(h + 1) * G].astype(np.float64)
            ref = o.scores(oq, qq, idx, b01, nn[s], gg[s])
            worst = max(worst, P.check_logits(logits[b, h * G:(h + 1) * G], ref, np.linalg.norm(qq, axis=1), nn[s], d))
    print("worst relative logit error", worst)


@pytest.mark.parametrize("nseq,n,bits", [(8, 8191, 3), (3, 40001, 4), (16, 4127, 2)])
def test_value_encoder_multi_tile_ragged(nseq, n, bits):
    """Values with more 64-token tiles than encoder workgroups (each
    workgroup loops over several tiles) and a partial last 32-token block;
    every code of every sequence is checked."""
    print(f"case: mse values nseq={nseq} n={n} bits={bits} tiles={nseq * -(-n // 64)}", flush=True)
    rng = np.random.default_rng(nseq * 7 + n)
    d = 128
    x = rng.standard_normal((nseq, n, d), dtype=np.float32)
    g = tq.Quantizer(d, bits, 0)
    oq = o.Quantizer(d, bits, 0)
    xt = torch.from_numpy(x).to(_dev()).bfloat16()
    codes, norms, _ = tq.tq_encode(g, tq.TQ_MSE, xt)
    torch.cuda.synchronize()
    xs = xt.float().cpu().numpy().astype(np.float64)
    cw = P.to_u32(codes)
    per = g.code_words(tq.TQ_MSE, 1, n)
    nn = norms.cpu().numpy()
    for s in range(nseq):
        P.check_mse_codes(oq, xs[s], cw[s * per:(s + 1) * per], nn[s * n:(s + 1) * n])
