"""Seeded synthetic workloads (inputs only; no quantisation arithmetic here).

Shapes and value distributions follow the five benchmark workloads of this
project.  All draws use numpy's PCG64 with a fixed data seed per workload;
bfloat16 inputs are produced by round-to-nearest-even from float32 and
returned both as raw uint16 bit patterns (for upload) and as float32 values
(for any CPU check).  Nothing here depends on the quantizer.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np


def bf16_round(x: np.ndarray):
    """float32 -> (uint16 bf16 bits, float32 value of those bits), RNE."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    vals = (r.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return r, vals


@dataclass
class Workload:
    name: str
    d: int
    bits: int
    arrays: dict = field(default_factory=dict)
    meta: dict = field(default_factory=dict)


def tiny(seed: int = 0, n: int = 4096, d: int = 128, nq: int = 16) -> Workload:
    """4096 fp32 keys, iid N(0,1), 4 distinct channels scaled x20; 16 fp32
    N(0,1) queries; 3 total bits."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, d), dtype=np.float32)
    ch = rng.choice(d, 4, replace=False)
    x[:, ch] *= np.float32(20.0)
    q = rng.standard_normal((nq, d), dtype=np.float32)
    return Workload("tiny-4096x128-b3", d, 3, {"x": x, "q": q}, {"outlier_channels": ch})


def decode_layer(bits: int, seed: int = 1, heads: int = 32, n: int = 8192, d: int = 128) -> Workload:
    """Single-layer decode: heads x n bf16 keys, N(0,1) per channel times a
    per-(head, channel) scale log-uniform in [1, 50]; one bf16 N(0,1) query
    per head."""
    rng = np.random.default_rng(seed)
    s = np.exp(rng.uniform(0.0, math.log(50.0), (heads, 1, d))).astype(np.float32)
    k = rng.standard_normal((heads, n, d), dtype=np.float32) * s
    kb, kv = bf16_round(k)
    qb, qv = bf16_round(rng.standard_normal((heads, d), dtype=np.float32))
    return Workload(f"decode-32x8192x128-b{bits}", d, bits,
                    {"k_bf16": kb, "k": kv, "q_bf16": qb, "q": qv})


def _gqa_tensors(rng, B, Hkv, Hq, N, d):
    """Values N(0,1); keys = random direction x rho[b,h] x ||v_t|| with rho
    log-uniform in [4, 182] per (batch, KV head); queries N(0, (3/rho)^2) so
    that logits / sqrt(d) have standard deviation about 3."""
    rho = np.exp(rng.uniform(math.log(4.0), math.log(182.0), (B, Hkv))).astype(np.float32)
    v = rng.standard_normal((B, Hkv, N, d), dtype=np.float32)
    vb, vv = bf16_round(v)
    del v
    dirs = rng.standard_normal((B, Hkv, N, d), dtype=np.float32)
    dirs /= np.linalg.norm(dirs, axis=-1, keepdims=True)
    dirs *= (rho[:, :, None, None] * np.linalg.norm(vv, axis=-1, keepdims=True))
    kb, kv = bf16_round(dirs)
    del dirs
    G = Hq // Hkv
    qs = np.repeat(3.0 / rho, G, axis=1)[:, :, None].astype(np.float32)
    q = rng.standard_normal((B, Hq, d), dtype=np.float32) * qs
    qb, qv = bf16_round(q)
    return {"k_bf16": kb, "k": kv, "v_bf16": vb, "v": vv, "q_bf16": qb, "q": qv, "rho": rho}


def gqa_layer(seed: int = 3, B: int = 8, Hkv: int = 8, Hq: int = 32, N: int = 32768, d: int = 128) -> Workload:
    """GQA decode layer: keys 3-bit (2-bit MSE + QJL), values 3-bit MSE."""
    rng = np.random.default_rng(seed)
    a = _gqa_tensors(rng, B, Hkv, Hq, N, d)
    return Workload(f"gqa-b{B}-kv{Hkv}-q{Hq}-n{N}-d{d}-b3", d, 3, a, {"B": B, "Hkv": Hkv, "Hq": Hq, "N": N})


def long_context(seed: int = 4, B: int = 1, Hkv: int = 8, Hq: int = 32, N: int = 131072, tail: int = 256,
                 d: int = 128) -> Workload:
    """Long context: 4-bit keys and values; the last `tail` tokens stay bf16."""
    rng = np.random.default_rng(seed)
    a = _gqa_tensors(rng, B, Hkv, Hq, N, d)
    return Workload(f"long-b{B}-kv{Hkv}-q{Hq}-n{N}-tail{tail}-d{d}-b4", d, 4, a,
                    {"B": B, "Hkv": Hkv, "Hq": Hq, "N": N, "tail": tail})


def vector_search(bits: int, seed: int = 5, n: int = 1_000_000, d: int = 200, nq: int = 1000,
                  chunk: int = 100_000) -> Workload:
    """Anisotropic Gaussian directions (variance 1/i on axis i) with
    log-normal norms (sigma 0.5); queries from the same law.  Stands in for a
    d = 200 word-embedding search set."""
    rng = np.random.default_rng(seed)
    sd = (1.0 / np.sqrt(np.arange(1, d + 1))).astype(np.float32)

    def draw(m):
        out = np.empty((m, d), dtype=np.float32)
        for s in range(0, m, chunk):
            e = min(m, s + chunk)
            g = rng.standard_normal((e - s, d), dtype=np.float32) * sd
            g /= np.linalg.norm(g, axis=1, keepdims=True)
            g *= rng.lognormal(0.0, 0.5, (e - s, 1)).astype(np.float32)
            out[s:e] = g
        return out

    x = draw(n)
    q = draw(nq)
    return Workload(f"search-{n}x{d}-q{nq}-b{bits}", d, bits, {"x": x, "q": q})
