"""Plain float64 CPU oracle for the TurboQuant hot path.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check of the entry module
and the CPU-baseline leg of the benchmark may import this module.  The product
path (the HIP library and its Python binding) never calls it, and this module
imports nothing from the product package.

Every function follows the web pages that describe TurboQuant; citations name
the page (by site and title) and the section on it:

  [hotdry]     blog.hotdry.top, "TurboQuant: vector-search compression" post
               sections "随机旋转与标量量化" (random rotation + scalar
               quantisation), "QJL 残差校正" (QJL residual correction),
               "工程配置参数清单" (engineering configuration),
               "精度调优与监控要点" (accuracy tuning and monitoring)
  [a2a]        a2a-mcp.org, "什麼是TurboQuant？" sections "第一階段：隨機旋轉 +
               PolarQuant 壓縮" (stage 1), "第二階段：QJL 殘差校正" (stage 2),
               "如何實作 TurboQuant" (how to implement)
  [friday]     friday-blog, "TurboQuant 深度解析（二）" sections
               "1. 三步壓縮的數學細節" (three-step maths), "2. 理論下界的意義"
               (lower bound)
  [wiselychen] ai-coding.wiselychen.com, "Google TurboQuant：KV Cache 壓縮 6x
               的技術突破…" section "最猛的社群實作：TurboQuant+"

Where the pages leave a step open the plainest reading is taken; each reading
is listed in the design notes of the repository (R-numbers below).

Notation: d = head dimension, b = total bits, b' = MSE bits (b-1 for keys in
"prod" mode, b for values in "mse" mode), K = 2**b' levels, m = QJL rows
(m = d unless a test asks otherwise), n = ||x||, u = x / n, y = Pi u.

Parity status: every function below is pinned by tests/test_oracle_*.py
against closed forms, brute force, textbook values or the pages' numbers,
except the bit layout of the packed record (pack_*/unpack_*), which the pages
do not define: it is pinned only by round-trip and size checks
("parity unpinned" as far as the pages go).
"""
from __future__ import annotations

import math

import numpy as np
from scipy import special

# ---------------------------------------------------------------------------
# 1. Random numbers the method draws (R: the pages name no generator).
#    SplitMix64 (Steele, Lea & Flood, OOPSLA 2014) is counter based: output k
#    of a stream started at state s is mix(s + (k+1)*GAMMA).  Uniforms take
#    the top 53 bits, offset by half a unit so that 0 and 1 never occur;
#    normals come from the Box-Muller transform (Box & Muller, 1958) applied
#    to consecutive uniform pairs.
# ---------------------------------------------------------------------------
GAMMA = np.uint64(0x9E3779B97F4A7C15)
MIX1 = np.uint64(0xBF58476D1CE4E5B9)
MIX2 = np.uint64(0x94D049BB133111EB)
TAG_ROTATION = 1   # stream that fills the Gaussian matrix G whose QR gives Pi
TAG_QJL = 2        # stream that fills the QJL matrix S
TAG_SIGNS = 3      # stream of the random signs of the structured (Hadamard) rotation


def splitmix64(state: int, n: int) -> np.ndarray:
    """First n outputs of SplitMix64 started at `state` (uint64 array)."""
    with np.errstate(over="ignore"):
        k = np.arange(1, n + 1, dtype=np.uint64)
        z = np.uint64(state) + k * GAMMA
        z = (z ^ (z >> np.uint64(30))) * MIX1
        z = (z ^ (z >> np.uint64(27))) * MIX2
        return z ^ (z >> np.uint64(31))


def stream_state(seed: int, tag: int) -> int:
    """Start state of the stream `tag` for quantizer seed `seed`."""
    return (int(seed) ^ (int(tag) << 56)) & 0xFFFFFFFFFFFFFFFF


def uniforms(state: int, n: int) -> np.ndarray:
    z = splitmix64(state, n)
    return ((z >> np.uint64(11)).astype(np.float64) + 0.5) * 2.0 ** -53


def normals(seed: int, tag: int, n: int) -> np.ndarray:
    """n standard normals of stream (seed, tag), Box-Muller on uniform pairs."""
    npairs = (n + 1) // 2
    u = uniforms(stream_state(seed, tag), 2 * npairs).reshape(npairs, 2)
    r = np.sqrt(-2.0 * np.log(u[:, 0]))
    t = 2.0 * math.pi * u[:, 1]
    out = np.empty((npairs, 2))
    out[:, 0] = r * np.cos(t)
    out[:, 1] = r * np.sin(t)
    return out.reshape(-1)[:n]


# ---------------------------------------------------------------------------
# 2. Random orthogonal rotation Pi: QR of a Gaussian matrix ([a2a] stage 1,
#    step 1; [hotdry] random rotation section).  R5: the sign of each column
#    of Q is fixed so that R has a positive diagonal, which makes the factor
#    unique (and Haar distributed).
# ---------------------------------------------------------------------------
def rotation(d: int, seed: int) -> np.ndarray:
    g = normals(seed, TAG_ROTATION, d * d).reshape(d, d)
    q, r = np.linalg.qr(g)
    return q * np.sign(np.diag(r))[None, :]


def rademacher_signs(seed: int, d: int) -> np.ndarray:
    """d random signs: output i of stream (seed, TAG_SIGNS) gives -1 when its
    top bit is set, +1 otherwise."""
    z = splitmix64(stream_state(seed, TAG_SIGNS), d)
    return np.where((z >> np.uint64(63)) == np.uint64(1), -1.0, 1.0)


def hadamard(d: int) -> np.ndarray:
    """Sylvester-Hadamard matrix of order d (a power of two):
    H[i, j] = (-1)^popcount(i & j)."""
    if d < 1 or d & (d - 1):
        raise ValueError("Hadamard order must be a power of two")
    i = np.arange(d)
    bits = np.bitwise_and(i[:, None], i[None, :])
    pop = np.zeros_like(bits)
    while bits.any():
        pop += bits & 1
        bits >>= 1
    return np.where(pop % 2 == 0, 1.0, -1.0)


def rotation_hadamard(d: int, seed: int) -> np.ndarray:
    """Structured rotation Pi = H D / sqrt(d), D = diag(random signs)
    ([wiselychen] community implementation section: a Walsh-Hadamard
    rotation in place of the dense one, bringing the rotated coordinates
    close to Gaussian).  Reading: one randomized Hadamard transform (signs
    on the input side, Sylvester order), for d a power of two."""
    return hadamard(d) * rademacher_signs(seed, d)[None, :] / math.sqrt(d)


def qjl_matrix(m: int, d: int, seed: int) -> np.ndarray:
    """S in R^{m x d}, iid N(0,1) entries ([hotdry] QJL section)."""
    return normals(seed, TAG_QJL, m * d).reshape(m, d)


# ---------------------------------------------------------------------------
# 3. Codebooks.  After rotation a coordinate of a unit vector follows the law
#    with density f(x) = C (1-x^2)^((d-3)/2) on [-1, 1], i.e. (x+1)/2 is
#    Beta((d-1)/2, (d-1)/2) ([a2a] stage 1; [hotdry] random rotation
#    section).  The codebook is the Lloyd-Max quantizer of that law
#    ([hotdry]: b-1 bits for the MSE stage of keys; [a2a]: Lloyd-Max on the
#    Beta law).
# ---------------------------------------------------------------------------
def beta_density(x, d: int):
    x = np.asarray(x, dtype=np.float64)
    c = math.exp(math.lgamma(d / 2.0) - math.lgamma((d - 1) / 2.0)) / math.sqrt(math.pi)
    return c * np.clip(1.0 - x * x, 0.0, None) ** ((d - 3) / 2.0)


def beta_cdf(x, d: int):
    a = (d - 1) / 2.0
    return special.betainc(a, a, (np.clip(np.asarray(x, dtype=np.float64), -1.0, 1.0) + 1.0) / 2.0)


def beta_partial_moment(lo, hi, d: int):
    """Integral of x f(x) over [lo, hi]; d/dx (1-x^2)^((d-1)/2) = -(d-1) x (1-x^2)^((d-3)/2)."""
    c = math.exp(math.lgamma(d / 2.0) - math.lgamma((d - 1) / 2.0)) / math.sqrt(math.pi)
    e = (d - 1) / 2.0
    lo = np.asarray(lo, dtype=np.float64)
    hi = np.asarray(hi, dtype=np.float64)
    return c * (np.clip(1 - lo * lo, 0, None) ** e - np.clip(1 - hi * hi, 0, None) ** e) / (d - 1)


def lloyd_max(d: int, levels: int, tol: float = 1e-14, max_iter: int = 200000):
    """Lloyd-Max fixed point for the rotated-coordinate law.

    Alternates the two optimality conditions: thresholds at the midpoints of
    neighbouring centroids, centroids at the conditional means of their cells.
    Returns (centroids[K], thresholds[K-1]), both ascending; the codebook is
    symmetrised (the law is symmetric and the fixed point unique, since the
    density is log-concave for d >= 3).
    """
    if d < 3:
        raise ValueError("d >= 3 required")
    sd = 1.0 / math.sqrt(d)
    a = (d - 1) / 2.0
    # start from the cell mid-quantiles of the law
    c = 2.0 * special.betaincinv(a, a, (np.arange(levels) + 0.5) / levels) - 1.0
    for _ in range(max_iter):
        t = 0.5 * (c[1:] + c[:-1])
        edges = np.concatenate(([-1.0], t, [1.0]))
        mass = np.diff(beta_cdf(edges, d))
        mom = beta_partial_moment(edges[:-1], edges[1:], d)
        c_new = mom / mass
        delta = np.max(np.abs(c_new - c))
        c = c_new
        if delta < tol * sd:
            break
    c = 0.5 * (c - c[::-1])
    t = 0.5 * (c[1:] + c[:-1])
    if levels % 2 == 0:
        t[levels // 2 - 1] = 0.0
    return c, t


def codebook_distortion(d: int, c: np.ndarray, t: np.ndarray) -> float:
    """Expected ||u - u_hat||^2 for a uniform unit vector u (all d coordinates).

    Per coordinate E[x^2] = 1/d, and at a Lloyd-Max point the cell means are
    the centroids, so the error is 1/d - sum_k c_k^2 P_k; times d.
    """
    edges = np.concatenate(([-1.0], t, [1.0]))
    mass = np.diff(beta_cdf(edges, d))
    return float(1.0 - d * np.sum(c * c * mass))


# ---------------------------------------------------------------------------
# 4. Quantizer state: (d, bits, seed) fixes everything (offline precompute,
#    [a2a] "how to implement", step 2).
# ---------------------------------------------------------------------------
class Quantizer:
    def __init__(self, d: int, bits: int, seed: int = 0, m: int | None = None, rotation_kind: str = "haar"):
        if not (3 <= d <= 1024):
            raise ValueError("d out of range")
        if not (1 <= bits <= 4):
            raise ValueError("bits out of range")
        self.d, self.bits, self.seed = d, bits, seed
        self.m = d if m is None else m
        self.rotation_kind = rotation_kind
        if rotation_kind == "haar":
            self.pi = rotation(d, seed)
        elif rotation_kind == "hadamard":
            self.pi = rotation_hadamard(d, seed)
        else:
            raise ValueError("rotation_kind must be 'haar' or 'hadamard'")
        self.s = qjl_matrix(self.m, d, seed)
        # keys ("prod"): b-1 MSE bits + 1 QJL bit; values ("mse"): b MSE bits
        self.bp_prod = bits - 1
        self.bp_mse = bits
        self.cb = {}
        for bp in {self.bp_prod, self.bp_mse}:
            if bp >= 1:
                self.cb[bp] = lloyd_max(d, 2 ** bp)

    def codebook(self, mode: str):
        bp = self.bp_prod if mode == "prod" else self.bp_mse
        if bp < 1:
            raise ValueError("prod mode needs bits >= 2")
        return bp, self.cb[bp][0], self.cb[bp][1]


# ---------------------------------------------------------------------------
# 5. Encode ([a2a] stage 1 and 2; [hotdry] both stages; [friday] step 1-3).
#    normalise -> rotate -> per-coordinate nearest centroid (threshold count,
#    R6: a value equal to a threshold takes the lower index) -> residual
#    r = x - x_hat -> sign(S r) with sign(0) = +1 (R7), gamma = ||r||.
# ---------------------------------------------------------------------------
def _rotate(qz: Quantizer, x: np.ndarray):
    x = np.asarray(x, dtype=np.float64)
    n = np.linalg.norm(x, axis=1)
    safe = np.where(n > 0, n, 1.0)
    u = np.where(n[:, None] > 0, x / safe[:, None], 0.0)   # R8: zero vector -> u = 0
    y = u @ qz.pi.T
    return x, n, y


def bucketize(y: np.ndarray, t: np.ndarray) -> np.ndarray:
    """idx = #{k : t_k < y}."""
    return np.sum(y[..., None] > t, axis=-1).astype(np.int64)


def encode_mse(qz: Quantizer, x: np.ndarray):
    """Returns (idx[n, d], norms[n]); values ("mse" mode, b bits, no QJL)."""
    bp, c, t = qz.codebook("mse")
    _, n, y = _rotate(qz, x)
    return bucketize(y, t), n


def mse_reconstruct(qz: Quantizer, mode: str, idx: np.ndarray, norms: np.ndarray):
    """x_hat = n * Pi^T c[idx]."""
    _, c, _ = qz.codebook(mode)
    return norms[:, None] * (c[idx] @ qz.pi)


def encode_prod(qz: Quantizer, x: np.ndarray):
    """Returns (idx[n, d], qjl_bits[n, m] in {0,1}, norms[n], gammas[n]) for keys."""
    bp, c, t = qz.codebook("prod")
    x, n, y = _rotate(qz, x)
    idx = bucketize(y, t)
    r = x - mse_reconstruct(qz, "prod", idx, n)
    gam = np.linalg.norm(r, axis=1)
    z = r @ qz.s.T
    return idx, (z >= 0).astype(np.uint8), n, gam


def qjl_from_indices(qz: Quantizer, x: np.ndarray, idx: np.ndarray):
    """Residual sketch recomputed from given MSE indices (parity cascade rule)."""
    x = np.asarray(x, dtype=np.float64)
    n = np.linalg.norm(x, axis=1)
    r = x - mse_reconstruct(qz, "prod", idx, n)
    z = r @ qz.s.T
    return (z >= 0).astype(np.uint8), np.linalg.norm(r, axis=1), z


# ---------------------------------------------------------------------------
# 6. Decode and scores ([hotdry] QJL section: x_tilde = x_hat + gamma *
#    sqrt(pi/2)/m * S^T sign(S r); R1: the page prints /d, the unbiased
#    constant is /m, identical when m = d).  The score is <q, x_tilde>
#    evaluated in the rotated domain from the indices, with the query
#    rotated and projected once ([a2a] stage 2 and "how to implement").
# ---------------------------------------------------------------------------
def qjl_scale(m: int) -> float:
    return math.sqrt(math.pi / 2.0) / m


def decode_prod(qz: Quantizer, idx, bits01, norms, gammas):
    sig = 2.0 * np.asarray(bits01, dtype=np.float64) - 1.0
    return mse_reconstruct(qz, "prod", idx, norms) + (gammas * qjl_scale(qz.m))[:, None] * (sig @ qz.s)


def decode_mse(qz: Quantizer, idx, norms):
    return mse_reconstruct(qz, "mse", idx, norms)


def scores(qz: Quantizer, q, idx, bits01, norms, gammas):
    """Logits[Q, N] = n <Pi q, c[idx]> + gamma sqrt(pi/2)/m <S q, sigma>."""
    _, c, _ = qz.codebook("prod")
    q = np.asarray(q, dtype=np.float64)
    q_rot = q @ qz.pi.T
    q_prj = q @ qz.s.T
    sig = 2.0 * np.asarray(bits01, dtype=np.float64) - 1.0
    mse = (c[idx] @ q_rot.T).T * norms[None, :]
    qjl = (sig @ q_prj.T).T * (gammas * qjl_scale(qz.m))[None, :]
    return mse + qjl


def scores_gqa(qz: Quantizer, q, idx, bits01, norms, gammas):
    """q [B, Hq, d]; idx [B, Hkv, N, d]; bits [B, Hkv, N, m]; norms/gammas
    [B, Hkv, N] -> logits [B, Hq, N].  R14: query head h reads KV head
    h // (Hq // Hkv)."""
    B, Hq, _ = q.shape
    Hkv = idx.shape[1]
    g = Hq // Hkv
    out = np.empty((B, Hq, idx.shape[2]))
    for b in range(B):
        for h in range(Hkv):
            out[b, h * g:(h + 1) * g] = scores(qz, q[b, h * g:(h + 1) * g], idx[b, h],
                                               bits01[b, h], norms[b, h], gammas[b, h])
    return out


def scores_mse(qz: Quantizer, q, idx, norms):
    """MSE-only keys ([hotdry] accuracy tuning section: a mode without the
    QJL correction, which can rank better in some settings): all b bits go to
    the Lloyd-Max index and the logit is n <Pi q, c[idx]> = <q, decode_mse>."""
    _, c, _ = qz.codebook("mse")
    q_rot = np.asarray(q, dtype=np.float64) @ qz.pi.T
    return (c[idx] @ q_rot.T).T * np.asarray(norms, dtype=np.float64)[None, :]


# ---------------------------------------------------------------------------
# 7. Decode attention over the packed cache (R13: the pages do not spell the
#    softmax out; the standard scaled dot product is taken, scale 1/sqrt(d)
#    unless the caller passes another, max-subtracted).  The most recent
#    tokens may be kept uncompressed ([hotdry] engineering configuration:
#    recent 128-256 tokens in full precision); their logits are exact dot
#    products and their values exact.
# ---------------------------------------------------------------------------
def attend(kq: Quantizer, vq: Quantizer, q, k_idx, k_bits, k_norms, k_gammas,
           v_idx, v_norms, k_tail=None, v_tail=None, scale=None):
    """q [Hg, d] queries of one KV head; compressed keys/values [N, ...];
    tails [T, d] (float).  Returns out [Hg, d].  k_bits = None: MSE-only keys
    (logits from scores_mse)."""
    q = np.asarray(q, dtype=np.float64)
    d = q.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    if k_bits is None:
        logit = scores_mse(kq, q, k_idx, k_norms)
    else:
        logit = scores(kq, q, k_idx, k_bits, k_norms, k_gammas)
    vals = decode_mse(vq, v_idx, v_norms)
    if k_tail is not None and len(k_tail):
        logit = np.concatenate([logit, q @ np.asarray(k_tail, dtype=np.float64).T], axis=1)
        vals = np.concatenate([vals, np.asarray(v_tail, dtype=np.float64)], axis=0)
    s = scale * logit
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=1, keepdims=True)
    return p @ vals


def sparse_v_dropset(kq: Quantizer, vq: Quantizer, q, k_idx, k_bits, k_norms, k_gammas, v_idx, v_norms,
                     v_threshold, k_tail=None, v_tail=None, scale=None, margin=1.0):
    """Sparse V ([wiselychen] TurboQuant+ table: the value work of low-weight
    tokens is skipped).  Reading (R26): the weight of compressed token t is
    w_t = p_t n_t, its softmax weight times its value norm (the size of its
    term in the output), and a token may leave the value sum when w_t is
    below v_threshold times the largest weight; its p_t stays in the
    normaliser.  Returns (p [Hg, N + T] normalised softmax weights, D [Hg, N]
    boolean: w_t < margin * v_threshold * max_u w_u over compressed u).  An
    implementation that compares against a running maximum drops a subset of
    D, since a running maximum never exceeds the overall one."""
    q = np.asarray(q, dtype=np.float64)
    d = q.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    if k_bits is None:
        logit = scores_mse(kq, q, k_idx, k_norms)
    else:
        logit = scores(kq, q, k_idx, k_bits, k_norms, k_gammas)
    n_comp = logit.shape[1]
    if k_tail is not None and len(k_tail):
        logit = np.concatenate([logit, q @ np.asarray(k_tail, dtype=np.float64).T], axis=1)
    s = scale * logit
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    w = p[:, :n_comp] * np.asarray(v_norms, dtype=np.float64)[None, :]
    wmax = w.max(axis=1, keepdims=True) if n_comp else np.zeros((len(q), 1))
    return p, w < margin * v_threshold * wmax


def sparse_v_bound(kq: Quantizer, vq: Quantizer, q, k_idx, k_bits, k_norms, k_gammas, v_idx, v_norms,
                   v_threshold, k_tail=None, v_tail=None, scale=None, margin=1.0):
    """Largest change of each output element [Hg, d] that dropping any subset
    of the set D of sparse_v_dropset from the value sum can cause:
    sum_{t in D} p_t |v_t[e]| (p normalised over all tokens), by the triangle
    inequality on out = sum_t p_t v_t."""
    p, D = sparse_v_dropset(kq, vq, q, k_idx, k_bits, k_norms, k_gammas, v_idx, v_norms, v_threshold,
                            k_tail, v_tail, scale, margin)
    vals = decode_mse(vq, v_idx, v_norms)
    n_comp = D.shape[1]
    return (p[:, :n_comp] * D) @ np.abs(vals)


def attend_segments(segments, q, k_tail=None, v_tail=None, scale=None):
    """Decode attention over a cache kept in several compressed segments
    (temporal decay, [wiselychen] TurboQuant+ table: older tokens are kept at
    a lower precision).  Reading (R28): each segment holds its own key and
    value quantizers and codes; the logits of all compressed tokens (each
    segment's keys scored with its own quantizer) and of the exact tail share
    one softmax, and the output sums every token's decoded value.

    segments: list of (kq, vq, k_idx, k_bits or None, k_norms, k_gammas, v_idx,
    v_norms); q [Hg, d]; tails [T, d].  Returns out [Hg, d]."""
    q = np.asarray(q, dtype=np.float64)
    d = q.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    logits, vals = [], []
    for (kq, vq, k_idx, k_bits, k_norms, k_gammas, v_idx, v_norms) in segments:
        if len(k_idx) == 0:
            continue
        if k_bits is None:
            logits.append(scores_mse(kq, q, k_idx, k_norms))
        else:
            logits.append(scores(kq, q, k_idx, k_bits, k_norms, k_gammas))
        vals.append(decode_mse(vq, v_idx, v_norms))
    if k_tail is not None and len(k_tail):
        logits.append(q @ np.asarray(k_tail, dtype=np.float64).T)
        vals.append(np.asarray(v_tail, dtype=np.float64))
    logit = np.concatenate(logits, axis=1)
    s = scale * logit
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=1, keepdims=True)
    return p @ np.concatenate(vals, axis=0)


def requantize(q_from: Quantizer, q_to: Quantizer, mode: str, idx, bits01, norms, gammas):
    """A token moving to an older, lower-precision segment (R28): its
    reconstruction at the old width -- x~ (MSE part plus the QJL term) for
    prod keys, x^ for values and MSE-only keys -- is encoded again with the new
    quantizer.  mode: "prod", "mse" (values) or "mse_keys".  Returns what
    encode_prod / encode_mse return for the new quantizer."""
    if mode == "prod":
        x = decode_prod(q_from, idx, bits01, norms, gammas)
        return encode_prod(q_to, x)
    x = decode_mse(q_from, idx, norms)
    return encode_mse(q_to, x)


def kv_width_config(width: float):
    """Fractional cache widths (R27, [hotdry] engineering configuration:
    "3.5-bit = 3-bit MSE + 1-bit QJL", 2.5-bit the more aggressive setting;
    [friday] comparison table: lowest width 2.5 bits): the width is the mean
    over the cached key and value coordinates.  Keys are coded with b_k - 1
    index bits plus one QJL bit, values with b_v index bits, and
    (b_k + b_v) / 2 = width with b_k = b_v + 1 for a half-integer width.
    Returns (key bits b_k, value bits b_v)."""
    w2 = round(2 * width)
    if abs(2 * width - w2) > 1e-9 or not 3 <= w2 <= 8:
        raise ValueError("width must be a multiple of 0.5 in [1.5, 4]")
    if w2 % 2 == 0:
        return w2 // 2, w2 // 2
    return (w2 + 1) // 2, (w2 - 1) // 2


# ---------------------------------------------------------------------------
# 8. Top-k by score (vector search with codes, [a2a] benchmark section on
#    GloVe-style search): order by (score descending, index ascending).
# ---------------------------------------------------------------------------
def topk(logits, k: int):
    logits = np.asarray(logits)
    out_i = np.empty((logits.shape[0], k), dtype=np.int64)
    out_s = np.empty((logits.shape[0], k))
    for r in range(logits.shape[0]):
        order = np.lexsort((np.arange(logits.shape[1]), -logits[r]))[:k]
        out_i[r] = order
        out_s[r] = logits[r, order]
    return out_s, out_i


# ---------------------------------------------------------------------------
# 9. Packed layout (ours; the pages fix only the bit budget: b' index bits +
#    1 QJL bit per coordinate, plus the norms, [hotdry] QJL section).
#
#    prod (keys), token major: uint32 words [N][G][b'+1] with G = ceil(d/32)
#      groups of 32 coordinates; word (g, p) holds bit p of the index of
#      coordinates 32g..32g+31 (bit i <-> coordinate 32g+i) for p < b', and
#      the QJL bits of rows 32g..32g+31 for p = b' (m = d).  Unused bits 0.
#    mse keys, token major: uint32 [N][G][b] (the prod layout without the
#      QJL plane, b = all bits to the index); norms only.
#    mse (values), 32-token blocks, coordinate major: uint32 words
#      [ceil(N/32)][b'][d]; word (blk, p, j) holds bit p of the index of
#      coordinate j of tokens 32blk..32blk+31 (bit i <-> token 32blk+i).
# ---------------------------------------------------------------------------
def _bits_to_words(bits: np.ndarray) -> np.ndarray:
    """bits [..., 32*W] in {0,1} -> uint32 [..., W], bit i of word w = bits[32w+i]."""
    sh = bits.shape
    b = bits.reshape(sh[:-1] + (sh[-1] // 32, 32)).astype(np.uint64)
    w = np.sum(b << np.arange(32, dtype=np.uint64), axis=-1)
    return w.astype(np.uint32)


def _words_to_bits(words: np.ndarray) -> np.ndarray:
    w = words.astype(np.uint64)[..., None]
    b = (w >> np.arange(32, dtype=np.uint64)) & np.uint64(1)
    return b.reshape(words.shape[:-1] + (words.shape[-1] * 32,)).astype(np.uint8)


def pack_prod(idx, bits01, bp: int, d: int) -> np.ndarray:
    n = idx.shape[0]
    G = (d + 31) // 32
    planes = np.zeros((n, bp + 1, G * 32), dtype=np.uint8)
    for p in range(bp):
        planes[:, p, :d] = (idx >> p) & 1
    planes[:, bp, :bits01.shape[1]] = bits01
    words = _bits_to_words(planes)              # [n, b'+1, G]
    return np.ascontiguousarray(words.transpose(0, 2, 1))  # [n, G, b'+1]


def unpack_prod(words, bp: int, d: int):
    words = np.asarray(words, dtype=np.uint32)
    n = words.shape[0]
    G = (d + 31) // 32
    w = words.reshape(n, G, bp + 1).transpose(0, 2, 1)
    planes = _words_to_bits(np.ascontiguousarray(w))   # [n, b'+1, 32G]
    idx = np.zeros((n, d), dtype=np.int64)
    for p in range(bp):
        idx |= planes[:, p, :d].astype(np.int64) << p
    return idx, planes[:, bp, :d].copy()


def pack_mse_keys(idx, bp: int, d: int) -> np.ndarray:
    """MSE-only keys, token major: uint32 [N][G][b'] (the prod layout without
    the QJL plane)."""
    n = idx.shape[0]
    G = (d + 31) // 32
    planes = np.zeros((n, bp, G * 32), dtype=np.uint8)
    for p in range(bp):
        planes[:, p, :d] = (idx >> p) & 1
    return np.ascontiguousarray(_bits_to_words(planes).transpose(0, 2, 1))


def unpack_mse_keys(words, bp: int, d: int):
    words = np.asarray(words, dtype=np.uint32)
    n = words.shape[0]
    G = (d + 31) // 32
    planes = _words_to_bits(np.ascontiguousarray(words.reshape(n, G, bp).transpose(0, 2, 1)))
    idx = np.zeros((n, d), dtype=np.int64)
    for p in range(bp):
        idx |= planes[:, p, :d].astype(np.int64) << p
    return idx


def pack_mse(idx, bp: int, d: int) -> np.ndarray:
    n = idx.shape[0]
    nb = (n + 31) // 32
    full = np.zeros((nb * 32, d), dtype=np.int64)
    full[:n] = idx
    out = np.zeros((nb, bp, d), dtype=np.uint32)
    blocks = full.reshape(nb, 32, d)
    for p in range(bp):
        bits = ((blocks >> p) & 1).transpose(0, 2, 1)    # [nb, d, 32 tokens]
        out[:, p, :] = _bits_to_words(bits)[..., 0]
    return out


def unpack_mse(words, n: int, bp: int, d: int):
    words = np.asarray(words, dtype=np.uint32)
    nb = (n + 31) // 32
    w = words.reshape(nb, bp, d)
    idx = np.zeros((nb, 32, d), dtype=np.int64)
    for p in range(bp):
        bits = _words_to_bits(w[:, p, :, None])     # [nb, d, 32]
        idx |= bits.transpose(0, 2, 1).astype(np.int64) << p
    return idx.reshape(nb * 32, d)[:n]


def record_bytes(mode: str, d: int, bits: int) -> int:
    """Bytes per vector including fp32 norm (and fp32 gamma for keys), R4."""
    G = (d + 31) // 32
    if mode == "prod":
        return 4 * G * bits + 8
    if mode == "mse_keys":
        return 4 * G * bits + 4
    return (bits * d) // 8 + 4
