"""Allocation-free decode attention (tq_attend_decode_noalloc, for callers
that cannot allocate device memory) against tq_attend_decode, the entry point
it mirrors, on the same inputs and through the C ABI.

Both run the same kernels with the same chunking, so the outputs must agree
bit for bit; each is also held to the attention tolerance against the oracle
on the GPU's codes.  Two calls in a row share the device's scratch array, the
second with a smaller input, so the second reads nothing the first left
behind.  A shape whose workspace exceeds the scratch is refused on the host.
"""
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


def _case(B, Hkv, Hq, N, tail, bits, seed, d=128):
    rng = np.random.default_rng(seed)
    a = W._gqa_tensors(rng, B, Hkv, Hq, N, d)
    k = _bf16(a["k_bf16"]).view(B * Hkv, N, d)
    v = _bf16(a["v_bf16"]).view(B * Hkv, N, d)
    q = _bf16(a["q_bf16"])
    n_comp = N - tail
    kq = tq.Quantizer(d, bits, 0)
    vq = tq.Quantizer(d, bits, 1)
    kc, kn, kg = tq.tq_encode(kq, tq.TQ_PROD, k[:, :n_comp].contiguous())
    vc, vn, _ = tq.tq_encode(vq, tq.TQ_MSE, v[:, :n_comp].contiguous())
    kt = k[:, n_comp:].contiguous().view(B, Hkv, tail, d) if tail else None
    vt = v[:, n_comp:].contiguous().view(B, Hkv, tail, d) if tail else None
    return dict(B=B, Hkv=Hkv, Hq=Hq, n_comp=n_comp, tail=tail, bits=bits, kq=kq, vq=vq, q=q, kc=kc, kn=kn, kg=kg,
                vc=vc, vn=vn, kt=kt, vt=vt, k=k, v=v, d=d)


def _oracle_check(c, out, groups):
    bits, n_comp, G, d = c["bits"], c["n_comp"], c["Hq"] // c["Hkv"], c["d"]
    ok, ov = o.Quantizer(d, bits, 0), o.Quantizer(d, bits, 1)
    kw, vw = P.to_u32(c["kc"]), P.to_u32(c["vc"])
    kn, kg, vn = (t.cpu().numpy().astype(np.float64) for t in (c["kn"], c["kg"], c["vn"]))
    qs = c["q"].float().cpu().numpy().astype(np.float64)
    kf, vf = c["k"].float().cpu().numpy().astype(np.float64), c["v"].float().cpu().numpy().astype(np.float64)
    perk, perv = c["kq"].code_words(tq.TQ_PROD, 1, n_comp), c["vq"].code_words(tq.TQ_MSE, 1, n_comp)
    for (b, h) in groups:
        s = b * c["Hkv"] + h
        ki, kb = o.unpack_prod(kw[s * perk:(s + 1) * perk].reshape(n_comp, -1), bits - 1, d)
        vi = o.unpack_mse(vw[s * perv:(s + 1) * perv], n_comp, bits, d)
        sl = slice(s * n_comp, (s + 1) * n_comp)
        tails = (kf[s, n_comp:], vf[s, n_comp:]) if c["tail"] else (None, None)
        ref = o.attend(ok, ov, qs[b, h * G:(h + 1) * G], ki, kb, kn[sl], kg[sl], vi, vn[sl], *tails)
        P.check_attention(out[b, h * G:(h + 1) * G], ref)


def _pair_of_calls(c):
    ref = tq.tq_attend_decode(c["kq"], c["vq"], c["q"], c["kc"], c["kn"], c["kg"], c["vc"], c["vn"], c["Hkv"],
                              c["n_comp"], c["kt"], c["vt"])
    out = torch.full_like(ref, float("nan"))
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    tq.tq_attend_decode_noalloc(c["kq"], c["vq"], c["q"], c["kc"], c["kn"], c["kg"], c["vc"], c["vn"], c["Hkv"],
                                c["n_comp"], c["kt"], c["vt"], out=out)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    return ref, out


def test_noalloc_matches_attend_decode_twice_then_smaller():
    print("case: noalloc call 1 B=4 Hkv=8 Hq=32 N=8192 tail=64 3-bit", flush=True)
    big = _case(4, 8, 32, 8192, 64, 3, seed=101)
    need = tq.attend_workspace_bytes(big["kq"], big["vq"], 4, 32, 8, big["n_comp"], 64)
    assert 0 < need <= tq.NOALLOC_SCRATCH_BYTES
    ref, out = _pair_of_calls(big)
    assert torch.equal(ref, out), float((ref - out).abs().max())
    _oracle_check(big, out.cpu().numpy(), [(0, 0), (3, 7)])
    print("case: noalloc call 2 (smaller) B=1 Hkv=2 Hq=8 N=777 tail=0 4-bit", flush=True)
    small = _case(1, 2, 8, 777, 0, 4, seed=102)
    ref2, out2 = _pair_of_calls(small)
    assert torch.equal(ref2, out2), float((ref2 - out2).abs().max())
    _oracle_check(small, out2.cpu().numpy(), [(0, 0), (0, 1)])
    print("case: noalloc call 3 (head dimension 256) B=1 Hkv=4 Hq=16 N=3000 tail=20 3-bit", flush=True)
    wide = _case(1, 4, 16, 3000, 20, 3, seed=103, d=256)
    ref3, out3 = _pair_of_calls(wide)
    assert torch.equal(ref3, out3), float((ref3 - out3).abs().max())
    _oracle_check(wide, out3.cpu().numpy(), [(0, 0), (0, 3)])


def test_noalloc_refuses_shapes_beyond_its_scratch():
    """32 x 8 KV heads x 32 query heads over 32768 tokens needs about 19 MB of
    workspace; the call is refused before any launch (the output keeps its
    contents), while tq_attend_decode with a workspace accepts the shape."""
    print("case: noalloc refuses B=32 Hkv=8 Hq=32 N=32768", flush=True)
    dev = _dev()
    B, Hkv, Hq, n = 32, 8, 32, 32768
    kq = tq.Quantizer(128, 3, 0)
    need = tq.attend_workspace_bytes(kq, kq, B, Hq, Hkv, n, 0)
    assert need > tq.NOALLOC_SCRATCH_BYTES
    nseq = B * Hkv
    kc = torch.zeros(kq.code_words(tq.TQ_PROD, nseq, n), dtype=torch.int32, device=dev)
    kn = torch.zeros(nseq * n, device=dev)
    kg = torch.zeros(nseq * n, device=dev)
    vc = torch.zeros(kq.code_words(tq.TQ_MSE, nseq, n), dtype=torch.int32, device=dev)
    vn = torch.zeros(nseq * n, device=dev)
    q = torch.zeros(B, Hq, 128, device=dev)
    out = torch.full((B, Hq, 128), 7.0, device=dev)
    with pytest.raises(tq.TQError) as e:
        tq.tq_attend_decode_noalloc(kq, kq, q, kc, kn, kg, vc, vn, Hkv, n, out=out)
    assert e.value.code == tq.TQ_EWORKSPACE and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
