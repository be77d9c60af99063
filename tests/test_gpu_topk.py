"""GPU parity: tq_scores with topk > 0 (fused top-k search) through the C ABI.

Each case checks the GPU's top k against the oracle's logits on identical
codes (tests/parity.py: set equality up to swaps within the logit tolerance
of the k-th score), and that the selection is exact on the GPU's own
scores: the top-k scores equal the full logits of tq_scores bit for bit and
are the k best of them under (score descending, index ascending)."""
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


def _exact_selection(logits, s, i):
    """s/i [Q, k] must be the k best of logits [Q, N] (float32) under
    (score desc, index asc), with the scores equal bit for bit."""
    k = i.shape[1]
    for r in range(logits.shape[0]):
        order = np.lexsort((np.arange(logits.shape[1]), -logits[r].astype(np.float64)))[:k]
        assert np.array_equal(order, i[r]), f"query {r}: selection differs from the exact top-{k} of the logits"
        assert np.array_equal(logits[r, order].view(np.uint32), s[r].view(np.uint32)), f"query {r}: score bits"


def _topk_case(d, bits, B, Hkv, Hq, n, topk, keys=None, seed=0, bf16=False):
    rng = np.random.default_rng(seed)
    g, oq = _pair(d, bits)
    if keys is None:
        keys = (rng.standard_normal((B * Hkv, n, d)) * (1.0 / np.sqrt(np.arange(1, d + 1)))).astype(np.float32)
    q = rng.standard_normal((B, Hq, d)).astype(np.float32)
    kt = torch.from_numpy(keys).to(_dev())
    qt = torch.from_numpy(q).to(_dev())
    if bf16:
        kt, qt = kt.bfloat16(), qt.bfloat16()
    codes, norms, gam = tq.tq_encode(g, tq.TQ_PROD, kt)
    s, i = tq.tq_scores(g, qt, codes, norms, gam, Hkv, n, topk=topk)
    full = tq.tq_scores(g, qt, codes, norms, gam, Hkv, n)
    torch.cuda.synchronize()
    s, i, full = s.cpu().numpy(), i.cpu().numpy(), full.cpu().numpy()
    cw = P.to_u32(codes)
    nn = norms.cpu().numpy().astype(np.float64)
    gg = gam.cpu().numpy().astype(np.float64)
    qs = qt.float().cpu().numpy().astype(np.float64)
    G = Hq // Hkv
    per = g.code_words(tq.TQ_PROD, 1, n)
    swaps = 0
    for b in range(B):
        for h in range(Hkv):
            sq = b * Hkv + h
            hs = slice(h * G, (h + 1) * G)
            _exact_selection(full[b, hs], s[b, hs], i[b, hs])
            idx, bits01 = o.unpack_prod(cw[sq * per:(sq + 1) * per].reshape(n, -1), bits - 1, d)
            kn = nn[sq * n:(sq + 1) * n]
            ref = o.scores(oq, qs[b, hs], idx, bits01, kn, gg[sq * n:(sq + 1) * n])
            swaps += P.check_topk(s[b, hs], i[b, hs], ref, np.linalg.norm(qs[b, hs], axis=1), kn, d)
    return swaps


@pytest.mark.parametrize("d,bits,B,Hkv,Hq,n,topk", [
    (200, 2, 1, 1, 40, 20000, 10),    # search shape: ragged row groups, many slices
    (200, 4, 1, 1, 40, 20000, 10),
    (200, 4, 1, 1, 17, 4099, 10),     # partial row tile, ragged last batch
    (128, 3, 2, 2, 6, 777, 5),        # GQA-shaped groups, 3 queries per key sequence
    (128, 3, 1, 4, 4, 1000, 1),       # one query per key sequence, top-1
    (64, 2, 1, 1, 9, 5000, 32),       # the 32-entry lists
    (64, 2, 1, 1, 9, 5000, 17),
    (48, 4, 1, 1, 3, 64, 16),
    (128, 3, 1, 2, 8, 3000, 13),      # the 16-entry lists above the 12-entry ones
    (16, 2, 1, 1, 5, 12, 12),         # k == n
])
def test_topk_shapes(d, bits, B, Hkv, Hq, n, topk):
    print(f"case: topk d={d} bits={bits} B={B} Hkv={Hkv} Hq={Hq} n={n} k={topk}", flush=True)
    swaps = _topk_case(d, bits, B, Hkv, Hq, n, topk)
    print("allowed swaps", swaps)


def test_topk_ties_go_to_lower_index():
    """Repeated keys give bit-identical scores; the lower index must win."""
    print("case: topk ties d=128 bits=3 n=3000 k=10", flush=True)
    rng = np.random.default_rng(11)
    base = rng.standard_normal((300, 128)).astype(np.float32)
    keys = np.concatenate([base] * 10)[None]   # key j repeats key j mod 300
    _topk_case(128, 3, 1, 1, 8, 3000, 10, keys=keys, seed=12)


def test_topk_ties_across_slices():
    """Keys repeat every 300 positions over 60000 keys, so equal best scores
    sit in many key slices: slices that see them late prune against a bound
    other slices published, and ties at that bound must survive (the lowest
    index wins)."""
    print("case: topk ties across slices d=128 bits=3 n=60000 k=10", flush=True)
    rng = np.random.default_rng(21)
    base = rng.standard_normal((300, 128)).astype(np.float32)
    keys = np.concatenate([base] * 200)[None]
    _topk_case(128, 3, 1, 1, 8, 60000, 10, keys=keys, seed=22)


@pytest.mark.parametrize("order", ["descending", "ascending"])
def test_topk_norm_ordered_keys(order):
    """Key norms sorted along the sequence: the best keys sit in the first
    (or last) slices, so the shared bound is high from the start (or only at
    the end) of the scan."""
    print(f"case: topk norm-ordered keys ({order}) d=200 bits=4 n=50000 k=10", flush=True)
    rng = np.random.default_rng(31)
    keys = rng.standard_normal((1, 50000, 200)).astype(np.float32)
    scale = np.geomspace(8.0, 0.125, 50000) if order == "descending" else np.geomspace(0.125, 8.0, 50000)
    keys *= scale[None, :, None].astype(np.float32)
    _topk_case(200, 4, 1, 1, 12, 50000, 10, keys=keys, seed=32)


@pytest.mark.parametrize("k", [1, 10, 12])
def test_topk_identical_keys(k):
    """Every key the same vector: all scores tie, so no key slice can bound
    what it leaves out below the k-th best and the search falls back to the
    exact scan for every query; the k lowest indices must come back."""
    print(f"case: topk identical keys d=200 bits=4 n=5000 k={k}", flush=True)
    rng = np.random.default_rng(41)
    keys = np.repeat(rng.standard_normal((1, 1, 200)).astype(np.float32), 5000, axis=1)
    _topk_case(200, 4, 1, 1, 9, 5000, k, keys=keys, seed=42)


def test_topk_block_of_best_keys():
    """A run of 40 copies of one strong key inside random keys: the slice
    holding the run cannot certify its k-th best (more than k equal bounds),
    other queries may; either way the lowest-indexed copies win."""
    print("case: topk block of best keys d=200 bits=4 n=30000 k=10", flush=True)
    rng = np.random.default_rng(51)
    keys = rng.standard_normal((1, 30000, 200)).astype(np.float32)
    keys[0, 12000:12040] = 6.0 * rng.standard_normal(200).astype(np.float32)
    _topk_case(200, 4, 1, 1, 12, 30000, 10, keys=keys, seed=52)


def test_topk_bf16_queries():
    print("case: topk bf16 d=128 bits=4 n=2500 k=10", flush=True)
    _topk_case(128, 4, 1, 2, 10, 2500, 10, bf16=True, seed=5)


@pytest.mark.parametrize("bits", [2, 4])
def test_search_full_size(bits):
    """Vector-search workload at full size: 1,000,000 keys of d = 200 encoded
    on the GPU, 1000 queries, top 10.  All queries: the top 10 is the exact
    selection over the GPU's own logits (checked on the GPU).  16 sampled
    queries: the top 10 against the oracle over all keys on identical codes."""
    print(f"case: search full size bits={bits}", flush=True)
    wl = W.vector_search(bits)
    g, oq = _pair(200, bits)
    n, nq, k = 1_000_000, 1000, 10
    xt = torch.from_numpy(wl.arrays["x"]).to(_dev())
    qt = torch.from_numpy(wl.arrays["q"][None]).to(_dev())
    codes, norms, gam = tq.tq_encode(g, tq.TQ_PROD, xt)
    s, i = tq.tq_scores(g, qt, codes, norms, gam, 1, n, topk=k)
    full = tq.tq_scores(g, qt, codes, norms, gam, 1, n)[0]
    s, i = s[0], i[0]
    # exact selection on the GPU's own scores, for every query
    assert torch.equal(full.gather(1, i), s), "top-k scores differ from the logits"
    kth = s[:, -1:]
    assert bool((s[:, :-1] >= s[:, 1:]).all())
    above = (full > kth).sum(dim=1)
    ties = (full == kth).sum(dim=1)
    sel_ties = (s == kth).sum(dim=1)
    assert bool((above + sel_ties == k).all()) and bool((ties >= sel_ties).all())
    # among keys tied with the k-th score, the selected ones are the lowest indices
    tied_rows = torch.nonzero(ties > sel_ties).flatten().tolist()
    for r in tied_rows:
        tied = torch.nonzero(full[r] == kth[r]).flatten()
        chosen = i[r][s[r] == kth[r]]
        assert torch.equal(tied[: chosen.numel()], torch.sort(chosen).values)
    del full
    # oracle on sampled queries
    rows = np.arange(0, nq, nq // 16)
    s_h, i_h = s.cpu().numpy()[rows], i.cpu().numpy()[rows]
    cw = P.to_u32(codes).reshape(n, -1)
    nn = norms.cpu().numpy().astype(np.float64)
    gg = gam.cpu().numpy().astype(np.float64)
    qs = wl.arrays["q"][rows].astype(np.float64)
    ref = np.empty((len(rows), n))
    for c0 in range(0, n, 100_000):
        c1 = min(n, c0 + 100_000)
        idx, bits01 = o.unpack_prod(cw[c0:c1], bits - 1, 200)
        ref[:, c0:c1] = o.scores(oq, qs, idx, bits01, nn[c0:c1], gg[c0:c1])
    swaps = P.check_topk(s_h, i_h, ref, np.linalg.norm(qs, axis=1), nn, 200)
    print("allowed swaps on sampled queries", swaps)
