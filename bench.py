"""Benchmark of the TurboQuant hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload gqa|long|decode|search]

One step = one pass of the whole hot path over one batch of synthetic input
already resident in HBM.  For the default workload (the GQA decode layer:
batch 8, 8 KV heads, 32 query heads, 32768 tokens, d = 128, 3-bit keys and
values) that is: encode the keys (prod codes) and values (mse codes),
rotate/project the queries, compute the logits from the packed keys, and run
decode attention (softmax . V) over the packed cache.  `long` is the same
step on the 131072-token cache with a 256-token bf16 tail (4-bit); `decode`
is encode + logits of the single-layer decode workload (32 heads x 8192
keys, one query per head); `search` is encode + fused top-10 of the
1,000,000 x 200 vector-search workload (1000 queries).

Printed: one JSON line.  For gqa/long/decode `value` is the packed-cache
bandwidth of the logits kernel (packed key bytes / kernel time); encode
keys/s and the attention kernel are reported beside it.  Kernel times come
from HIP events recorded on the stream the kernels run on (the library
launches on torch's current stream, where the events are recorded too), over
the timed steps.  Code buffers alternate between two copies so that every
scan reads codes written a full step (more than 1 GB of other traffic)
earlier, i.e. from HBM, not from the 256 MB last-level cache.

`roofline.traffic` is the HBM traffic of one logits launch measured with the
FETCH_SIZE and WRITE_SIZE counters (profiles/scores_kernel_gqa_traffic.txt,
each scaled by what the counter reads for a copy kernel of known size); it is
null when the kernel sources have changed since those counters were taken.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FP32_MFMA_PEAK_TFLOPS = 157.3
FP8_MFMA_PEAK_TFLOPS = 5000.0
FP16_MFMA_PEAK_TFLOPS = 2500.0
METRIC = "packed-KV logits GB/s (% of HBM peak) + encode keys/s, d=128 3-bit, 1 MI355X"
# sources whose compiled code the logits kernel is made of
SCORES_SOURCES = ["vector_quantization_tq_amd/csrc/tq_scores.hip", "vector_quantization_tq_amd/csrc/tq_device.h",
                  "vector_quantization_tq_amd/build.py"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "scores_kernel_gqa_traffic.txt")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="gqa", choices=["gqa", "long", "decode", "search", "decay"])
    ap.add_argument("--bits", type=int, default=None,
                    help="key bits (default: gqa 3, long 4, decode 3, search 4)")
    ap.add_argument("--key-mode", default="prod", choices=["prod", "mse"],
                    help="gqa/long: prod keys (b-1 MSE bits + QJL) or MSE-only keys (all b bits to the index)")
    ap.add_argument("--value-bits", type=int, default=None, help="gqa/long: value bits (default: the key bits)")
    ap.add_argument("--kv-width", type=float, default=None,
                    help="gqa/long: mean cache width in bits per key and value coordinate, a multiple of 0.5 "
                         "(3.5 = 4-bit prod keys, i.e. 3-bit index + 1 QJL bit, with 3-bit values); sets --bits and "
                         "--value-bits")
    ap.add_argument("--v-threshold", type=float, default=None,
                    help="gqa/long: sparse V (tq_attend_decode_sparse with this threshold in [0, 1))")
    ap.add_argument("--head-dim", type=int, default=128, choices=[64, 96, 128, 256],
                    help="gqa/long: head dimension d of the same layer shape (default 128)")
    ap.add_argument("--rotation", default="haar", choices=["haar", "hadamard"],
                    help="gqa/long: dense Haar rotation (QR of a Gaussian) or the structured H D / sqrt(d)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-baseline-all", action="store_true",
                    help="only time the oracle (no GPU): encode keys/s and logits GB/s of packed keys on a bounded "
                         "sample of each of the five workloads, with all host threads and with one; one JSON line "
                         "per workload and thread count")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a 256 MiB device copy 3 times (the known-size kernel for counter scaling)")
    ap.add_argument("--ceiling", action="store_true",
                    help="gqa: also time a plain streaming kernel that moves the logits scan's bytes (same buffers, "
                         "same read/write mix, no arithmetic) right after the scan in every step")
    return ap.parse_args()


def sources_sha256(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per logits launch from the counter summary, or None when it is
    missing or was taken on other kernel sources."""
    try:
        kv = {}
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("source_sha256") != sources_sha256(SCORES_SOURCES):
            return None
        return int(float(kv["traffic_bytes_per_launch"]))
    except (OSError, KeyError, ValueError):
        return None


def copy_calibration(torch, dev):
    x = torch.ones(64 << 20, dtype=torch.float32, device=dev)   # 256 MiB
    y = torch.empty_like(x)
    for _ in range(3):
        torch.neg(x, out=y)
    torch.cuda.synchronize()
    del x, y


def bf16_tensor(torch, u16, dev):
    import numpy as np
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).to(dev).view(torch.bfloat16)


class Timer:
    """Per-kernel HIP events on the stream the library launches on (torch's
    current stream).  The events are created without the system-scope fence
    (hipEventDisableSystemFence): a timing event then records its timestamp in
    stream order without flushing the caches for the host, so it does not add
    a cache write-back to the interval it brackets."""

    FLAGS = 0x20000000   # hipEventDisableSystemFence

    def __init__(self, torch):
        import ctypes
        self.torch = torch
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.pending = []
        self.acc = {}
        self.count = {}
        self.pool = []

    def _event(self):
        if self.pool:
            return self.pool.pop()
        e = self.ct.c_void_p()
        if self.hip.hipEventCreateWithFlags(self.ct.byref(e), self.ct.c_uint(self.FLAGS)) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        return e

    def mark(self):
        e = self._event()
        stream = self.ct.c_void_p(self.torch.cuda.current_stream().cuda_stream)
        if self.hip.hipEventRecord(e, stream) != 0:
            raise RuntimeError("hipEventRecord failed")
        return e

    def span(self, name, a, b):
        self.pending.append((name, a, b))

    def collect(self):
        ms = self.ct.c_float()
        for name, a, b in self.pending:
            if self.hip.hipEventElapsedTime(self.ct.byref(ms), a, b) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            self.acc[name] = self.acc.get(name, 0.0) + ms.value
            self.count[name] = self.count.get(name, 0) + 1
        seen = {}
        for _, a, b in self.pending:
            seen[a.value] = a
            seen[b.value] = b
        self.pool.extend(seen.values())
        self.pending = []

    def avg_ms(self, name):
        return self.acc[name] / self.count[name]


def cpu_baseline_gqa(wl, steps_note):
    """The oracle as it stands, on a bounded sample of the same workload."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import tq_oracle as o
    oq = o.Quantizer(128, 3, 0)
    # sample: the first 16384 keys of each of the first 4 (batch, KV head) groups
    nk = 16384
    keys = wl.arrays["k"][0, :4, :nk].reshape(-1, 128).astype(np.float64)
    qs = wl.arrays["q"][0, :16].astype(np.float64)        # the 4 query heads of each of the 4 groups
    t0 = time.perf_counter()
    idx, bits, nrm, gam = o.encode_prod(oq, keys)
    t1 = time.perf_counter()
    reps = 0
    t2 = time.perf_counter()
    while True:
        for h in range(4):
            sl = slice(h * nk, (h + 1) * nk)
            o.scores(oq, qs[4 * h:4 * h + 4], idx[sl], bits[sl], nrm[sl], gam[sl])
        reps += 1
        if time.perf_counter() - t2 > 10.0:
            break
    t3 = time.perf_counter()
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    packed = 4 * nk * o.record_bytes("prod", 128, 3)
    return {
        "value": packed * reps / (t3 - t2) / 1e9,
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"float64 numpy oracle: logits of 4 query heads x {nk} keys for 4 (batch, KV head) groups, "
                  f"{reps} passes in {t3 - t2:.1f} s; encode of the same {4 * nk} keys took {t1 - t0:.2f} s "
                  f"({4 * nk / (t1 - t0):.0f} keys/s)",
        "encode_keys_per_s": 4 * nk / (t1 - t0),
    }


def run_gqa(args, torch, dev, tq, wl_fn, name, bits, n_tail=0):
    import numpy as np
    wl = wl_fn()
    B, Hkv, Hq, N = wl.meta["B"], wl.meta["Hkv"], wl.meta["Hq"], wl.meta["N"]
    d = wl.d
    n_comp = N - n_tail
    k_all = bf16_tensor(torch, wl.arrays["k_bf16"], dev).view(B * Hkv, N, d)
    v_all = bf16_tensor(torch, wl.arrays["v_bf16"], dev).view(B * Hkv, N, d)
    q = bf16_tensor(torch, wl.arrays["q_bf16"], dev)
    k = k_all[:, :n_comp].contiguous()
    v = v_all[:, :n_comp].contiguous()
    k_tail = k_all[:, n_comp:].contiguous().view(B, Hkv, n_tail, d) if n_tail else None
    v_tail = v_all[:, n_comp:].contiguous().view(B, Hkv, n_tail, d) if n_tail else None
    mse_keys = args.key_mode == "mse"
    kmode = tq.TQ_MSE_KEYS if mse_keys else tq.TQ_PROD
    vbits = args.value_bits or bits
    rot = tq.TQ_ROT_HADAMARD if args.rotation == "hadamard" else tq.TQ_ROT_HAAR
    qz = tq.Quantizer(d, bits, 0, rot)
    if mse_keys:
        qz.set_key_mode(tq.TQ_MSE_KEYS)
    qv = qz if vbits == bits else tq.Quantizer(d, vbits, 0, rot)
    nseq = B * Hkv
    copies = []
    for _ in range(2):
        ck = torch.empty(qz.code_words(kmode, nseq, n_comp), dtype=torch.int32, device=dev)
        kn = torch.empty(nseq * n_comp, dtype=torch.float32, device=dev)
        kg = None if mse_keys else torch.empty(nseq * n_comp, dtype=torch.float32, device=dev)
        cv = torch.empty(qv.code_words(tq.TQ_MSE, nseq, n_comp), dtype=torch.int32, device=dev)
        vn = torch.empty(nseq * n_comp, dtype=torch.float32, device=dev)
        copies.append((ck, kn, kg, cv, vn))
    logits = torch.empty((B, Hq, n_comp), dtype=torch.float32, device=dev)
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    ws_s = torch.empty(tq.scores_workspace_bytes(qz, B, Hq, Hkv, n_comp), dtype=torch.uint8, device=dev)
    attend_ok = True
    try:
        ws_a = torch.empty(max(tq.attend_workspace_bytes(qz, qv, B, Hq, Hkv, n_comp, n_tail), 256), dtype=torch.uint8,
                           device=dev)
    except Exception:
        attend_ok = False
    stream_mix = None
    if args.ceiling:
        import ctypes
        if not (d == 128 and bits == 3 and not mse_keys and n_comp % 64 == 0):
            raise SystemExit("--ceiling: the streaming kernel mirrors 3-bit prod keys at d = 128, n a multiple of 64")
        slib = ctypes.CDLL(os.path.join(ROOT, "vector_quantization_tq_amd", "libtq_stream.so"))
        slib.tq_stream_scan_mix.restype = ctypes.c_int
        slib.tq_stream_scan_mix.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                            ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
        mix_out = torch.empty((nseq, n_comp, 4), dtype=torch.float32, device=dev)

        def stream_mix(c):
            rc = slib.tq_stream_scan_mix(ctypes.c_void_p(c[0].data_ptr()), ctypes.c_void_p(c[1].data_ptr()),
                                         ctypes.c_void_p(c[2].data_ptr()), n_comp, nseq,
                                         ctypes.c_void_p(mix_out.data_ptr()),
                                         ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
            if rc != 0:
                raise RuntimeError(f"tq_stream_scan_mix failed ({rc})")
    # fill both copies once
    for c in copies:
        tq.tq_encode(qz, kmode, k, out=(c[0], c[1], c[2]))
        tq.tq_encode(qv, tq.TQ_MSE, v, out=(c[3], c[4], None))
    mix_src = [(c[0].clone(), c[1].clone(), c[2].clone()) for c in copies] if stream_mix is not None else None
    if attend_ok:
        try:
            c = copies[0]
            tq.tq_attend_decode(qz, qv, q, c[0], c[1], c[2], c[3], c[4], Hkv, n_comp, k_tail, v_tail, 0.0, out=out,
                                workspace=ws_a, v_threshold=args.v_threshold)
        except tq.TQError:
            attend_ok = False
    torch.cuda.synchronize()

    timer = Timer(torch)

    def step(i, timed):
        w = copies[i % 2]          # written now
        r = copies[(i + 1) % 2]    # written one step ago
        e0 = timer.mark()
        tq.tq_encode(qz, kmode, k, out=(w[0], w[1], w[2]))
        e1 = timer.mark()
        tq.tq_encode(qv, tq.TQ_MSE, v, out=(w[3], w[4], None))
        e2 = timer.mark()
        tq.tq_query_prep(qz, q, Hkv, workspace=ws_s)
        e3 = timer.mark()
        tq.tq_scores_from_prep(qz, B, Hq, Hkv, r[0], r[1], r[2], n_comp, ws_s, out=logits)
        e4 = timer.mark()
        if attend_ok:
            tq.tq_attend_decode(qz, qv, q, r[0], r[1], r[2], r[3], r[4], Hkv, n_comp, k_tail, v_tail, 0.0, out=out,
                                workspace=ws_a, v_threshold=args.v_threshold)
        e5 = timer.mark()
        if stream_mix is not None:
            # its own code copies, alternating like the scan's: each is read
            # every other step, with more than 1 GB of other traffic between
            stream_mix(mix_src[i % 2])
            e6 = timer.mark()
            if timed:
                timer.span("stream_ceiling", e5, e6)
        if timed:
            timer.span("encode_keys", e0, e1)
            timer.span("encode_values", e1, e2)
            timer.span("query_prep", e2, e3)
            timer.span("scores", e3, e4)
            if attend_ok:
                timer.span("attend", e4, e5)

    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    timer.collect()

    nkeys = nseq * n_comp
    # packed key bytes per key: codes + norm (+ gamma for prod keys)
    rec_k = 4 * ((d + 31) // 32) * bits + (4 if mse_keys else 8)
    rec_v = (vbits * d) // 8 + 4                      # packed value bytes per token (codes + norm)
    G = Hq // Hkv
    scores_ms = timer.avg_ms("scores")
    scores_alg = nkeys * (rec_k + 4 * G)              # read packed keys, write fp32 logits
    packed_gbs = nkeys * rec_k / (scores_ms * 1e-3) / 1e9
    enc_ms = timer.avg_ms("encode_keys")
    enc_flop = nkeys * (2.0 if mse_keys else 4.0) * d * d   # Pi x (and S' rho for prod keys) per key
    res = {
        "metric": METRIC,
        "value": round(packed_gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round((t1 - t0) * 1e3 / args.steps, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8xfp4 MFMA, f32 accumulate",
        "data": "synthetic",
        "config": {"workload": name, "batch": B, "kv_heads": Hkv, "q_heads": Hq, "tokens": N, "tail_bf16": n_tail,
                   "d": d, "bits_keys": bits, "bits_values": vbits,
                   "key_mode": "mse-only (b MSE bits)" if mse_keys else "prod (b-1 MSE + 1 QJL)",
                   "rotation": args.rotation,
                   "kv_width_bits": (bits + vbits) / 2,
                   "value_mode": "mse" if args.v_threshold is None else f"mse, sparse V threshold {args.v_threshold}"},
        "packed_pct_of_hbm_peak": round(100 * packed_gbs / HBM_PEAK_GBS, 1),
        "encode_keys_per_s": round(nkeys / (enc_ms * 1e-3), 0),
        "kernels_ms": {k2: round(timer.avg_ms(k2), 4) for k2 in timer.acc},
        "tq_scores_call_gb_per_s": round(nkeys * rec_k / ((scores_ms + timer.avg_ms("query_prep")) * 1e-3) / 1e9, 1),
        "roofline": {
            "kernel": "scores_kernel (tq_scores_from_prep)",
            "bound": "hbm",
            "achieved": round(scores_alg / (scores_ms * 1e-3) / 1e9, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(scores_alg / (scores_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "traffic": (measured_traffic() if name.startswith("gqa") and not mse_keys and d == 128 and bits == 3
                        and args.rotation == "haar" else None),
            "algorithmic_bytes_per_launch": scores_alg,
            "bytes_per_key": rec_k + 4 * G,
        },
        "roofline_encode": {
            "kernel": "%s (tq_encode, %s)" % (
                ("encode_wht_kernel" if args.rotation == "hadamard" else "encode_tile_kernel") if mse_keys
                else ("encode_keys_split_kernel" if d == 128 else "encode_tile_kernel"),
                "mse keys" if mse_keys else "prod"),
            "bound": "mfma",
            "achieved": round(enc_flop / (enc_ms * 1e-3) / 1e12, 2),
            "peak": FP16_MFMA_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(enc_flop / (enc_ms * 1e-3) / 1e12 / FP16_MFMA_PEAK_TFLOPS, 4),
            "flop_per_key": (2 if mse_keys else 4) * d * d,
            "note": "algorithmic flop per key (4d^2 prod, 2d^2 mse keys); the fp16 MFMA runs hi/lo split operands, "
                    "2 products per rotation term (bf16 keys) and 3 per QJL term",
            "issued_frac": round((2.0 if mse_keys else 2.5) * enc_flop / (enc_ms * 1e-3) / 1e12
                                 / FP16_MFMA_PEAK_TFLOPS, 4),
        },
    }
    if "stream_ceiling" in timer.acc:
        cm = timer.avg_ms("stream_ceiling")
        res["stream_ceiling"] = {
            "kernel": "stream_scan_mix (libtq_stream.so): the scan's reads and writes, no arithmetic",
            "ms": round(cm, 4),
            "gb_per_s": round(scores_alg / (cm * 1e-3) / 1e9, 1),
            "frac_of_peak": round(scores_alg / (cm * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "scan_time_over_ceiling": round(scores_ms / cm, 3),
        }
    if attend_ok:
        at_ms = timer.avg_ms("attend")
        at_bytes = nkeys * (rec_k + rec_v) + (nseq * n_tail * d * 2 * 2)
        res["roofline_attend"] = {
            "kernel": "tq_attend_decode (all its launches)",
            "bound": "hbm",
            "achieved": round(at_bytes / (at_ms * 1e-3) / 1e9, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(at_bytes / (at_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "algorithmic_bytes_per_launch": at_bytes,
        }
    return res, wl


def _timed_loop(args, torch, step):
    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, True)
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def _common(args, ms_step, config, value, unit, metric=METRIC):
    return {"metric": metric, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(ms_step, 3), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "fp8xfp4 MFMA, f32 accumulate", "data": "synthetic", "config": config}


def run_decode(args, torch, dev, tq, W):
    """Single-layer decode: encode 32 x 8192 keys, then the logits of one query
    per head (the logits are launch-bound at this size)."""
    bits = args.bits or 3
    wl = W.decode_layer(bits)
    H, N, d = 32, 8192, 128
    k = bf16_tensor(torch, wl.arrays["k_bf16"], dev).view(H, N, d)
    q = bf16_tensor(torch, wl.arrays["q_bf16"], dev).view(1, H, d)
    qz = tq.Quantizer(d, bits, 0)
    copies = []
    for _ in range(2):
        copies.append((torch.empty(qz.code_words(tq.TQ_PROD, H, N), dtype=torch.int32, device=dev),
                       torch.empty(H * N, dtype=torch.float32, device=dev),
                       torch.empty(H * N, dtype=torch.float32, device=dev)))
        tq.tq_encode(qz, tq.TQ_PROD, k, out=copies[-1])
    logits = torch.empty((1, H, N), dtype=torch.float32, device=dev)
    ws = torch.empty(tq.scores_workspace_bytes(qz, 1, H, H, N), dtype=torch.uint8, device=dev)
    timer = Timer(torch)

    def step(i, timed):
        w, r = copies[i % 2], copies[(i + 1) % 2]
        e0 = timer.mark()
        tq.tq_encode(qz, tq.TQ_PROD, k, out=w)
        e1 = timer.mark()
        tq.tq_query_prep(qz, q, H, workspace=ws)
        e2 = timer.mark()
        tq.tq_scores_from_prep(qz, 1, H, H, r[0], r[1], r[2], N, ws, out=logits)
        e3 = timer.mark()
        if timed:
            timer.span("encode_keys", e0, e1)
            timer.span("query_prep", e1, e2)
            timer.span("scores", e2, e3)

    el = _timed_loop(args, torch, step)
    timer.collect()
    rec_k = 4 * ((d + 31) // 32) * bits + 8
    sc = timer.avg_ms("scores")
    enc = timer.avg_ms("encode_keys")
    gbs = H * N * rec_k / (sc * 1e-3) / 1e9
    res = _common(args, el * 1e3 / args.steps,
                  {"workload": f"decode-layer 32 heads x 8192 keys d128 {bits}-bit, 1 query per head"},
                  round(gbs, 1), "GB/s")
    res["encode_keys_per_s"] = round(H * N / (enc * 1e-3), 0)
    res["kernels_ms"] = {k2: round(timer.avg_ms(k2), 4) for k2 in timer.acc}
    res["roofline"] = {"kernel": "scores_kernel", "bound": "hbm",
                       "achieved": round(H * N * (rec_k + 4) / (sc * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBS,
                       "unit": "GB/s", "frac": round(H * N * (rec_k + 4) / (sc * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                       "traffic": None, "note": "launch-bound: the packed keys are %.1f MB" % (H * N * rec_k / 1e6)}
    return res


def run_search(args, torch, dev, tq, W):
    """Vector search: encode the 1,000,000 x 200 database, then the fused top-10
    of 1000 queries straight from the codes."""
    bits = args.bits or 4
    wl = W.vector_search(bits)
    n, d, nq, k = 1_000_000, 200, 1000, 10
    x = torch.from_numpy(wl.arrays["x"]).to(dev)
    q = torch.from_numpy(wl.arrays["q"][None]).to(dev)
    qz = tq.Quantizer(d, bits, 0)
    copies = []
    for _ in range(2):
        copies.append((torch.empty(qz.code_words(tq.TQ_PROD, 1, n), dtype=torch.int32, device=dev),
                       torch.empty(n, dtype=torch.float32, device=dev),
                       torch.empty(n, dtype=torch.float32, device=dev)))
        tq.tq_encode(qz, tq.TQ_PROD, x, out=copies[-1])
    out_s = torch.empty((1, nq, k), dtype=torch.float32, device=dev)
    out_i = torch.empty((1, nq, k), dtype=torch.int64, device=dev)
    ws = torch.empty(tq.scores_workspace_bytes(qz, 1, nq, 1, n, k), dtype=torch.uint8, device=dev)
    timer = Timer(torch)

    def step(i, timed):
        w, r = copies[i % 2], copies[(i + 1) % 2]
        e0 = timer.mark()
        tq.tq_encode(qz, tq.TQ_PROD, x, out=w)
        e1 = timer.mark()
        tq.tq_scores(qz, q, r[0], r[1], r[2], 1, n, topk=k, out=out_s, out_idx=out_i, workspace=ws)
        e2 = timer.mark()
        if timed:
            timer.span("encode_keys", e0, e1)
            timer.span("topk", e1, e2)

    el = _timed_loop(args, torch, step)
    timer.collect()
    # recall@10 of the codes against the exact float32 top 10 (context)
    exact = torch.topk(torch.matmul(q[0], x.t()), k, dim=1).indices
    got = out_i[0]
    recall = float((got[:, :, None] == exact[:, None, :]).any(dim=2).float().mean())
    tk = timer.avg_ms("topk")
    enc = timer.avg_ms("encode_keys")
    gw = (d + 31) // 32
    rec_k = 4 * gw * bits + 8
    alg_flop = 2.0 * n * nq * (d + d)                     # MSE and QJL inner products, m = d
    T = (1 << (bits - 2)) + 1
    # the bounded scan (k <= 12): one 16x16x128 MFMA per Walsh/QJL term and
    # 128 coordinates covers 16 keys x 8 queries (query limbs 0-1); the merge's
    # exact rescoring of a few candidates per query is left out
    issued = (nq + 7) // 8 * ((n + 15) // 16) * T * ((d + 127) // 128) * 2 * 16 * 16 * 128
    res = _common(args, el * 1e3 / args.steps,
                  {"workload": f"vector-search 1000000 x 200 fp32, 1000 queries, top-10, {bits}-bit"},
                  round(nq / (tk * 1e-3), 1), "queries/s", metric="top-10 queries/s from packed codes, 1 MI355X")
    res["scan_gb_per_s"] = round(n * rec_k / (tk * 1e-3) / 1e9, 1)
    res["encode_keys_per_s"] = round(n / (enc * 1e-3), 0)
    res["recall_at_10_vs_exact_fp32"] = round(recall, 4)
    res["kernels_ms"] = {k2: round(timer.avg_ms(k2), 4) for k2 in timer.acc}
    res["roofline"] = {"kernel": "topk_lb_scan_kernel + merges (tq_scores, topk=10)", "bound": "mfma",
                       "achieved": round(alg_flop / (tk * 1e-3) / 1e12, 2), "peak": FP8_MFMA_PEAK_TFLOPS,
                       "unit": "TFLOP/s", "frac": round(alg_flop / (tk * 1e-3) / 1e12 / FP8_MFMA_PEAK_TFLOPS, 4),
                       "traffic": None, "algorithmic_flop_per_launch": alg_flop,
                       "issued_mfma_flop_per_launch": issued,
                       "issued_mfma_tflops": round(issued / (tk * 1e-3) / 1e12, 1)}
    return res


def run_decay(args, torch, dev, tq, W):
    """Temporal decay on the long-context layer: the older two thirds of the
    130816 compressed tokens (87168, a multiple of 128) are kept at 2-bit
    keys and values, the newer 43648 at 4 bits, the last 256 in bf16.  A step
    encodes both segments, scores them (one scan per segment) and runs decode
    attention over the segmented cache with one softmax; beside it, the
    re-quantization of 8 x 4096 tokens from 4 to 2 bits (keys and values) is
    timed, the work of moving an aged block to the older segment."""
    wl = W.long_context()
    B, Hkv, Hq, N, tail, d = 1, 8, 32, 131072, 256, 128
    nseq = B * Hkv
    n_comp = N - tail
    n_old = (2 * n_comp // 3) // 128 * 128
    n_new = n_comp - n_old
    b_old, b_new = 2, 4
    k_all = bf16_tensor(torch, wl.arrays["k_bf16"], dev).view(nseq, N, d)
    v_all = bf16_tensor(torch, wl.arrays["v_bf16"], dev).view(nseq, N, d)
    q = bf16_tensor(torch, wl.arrays["q_bf16"], dev)
    parts = {"old": (k_all[:, :n_old].contiguous(), v_all[:, :n_old].contiguous(), n_old, tq.Quantizer(d, b_old, 0)),
             "new": (k_all[:, n_old:n_comp].contiguous(), v_all[:, n_old:n_comp].contiguous(), n_new,
                     tq.Quantizer(d, b_new, 0))}
    k_tail = k_all[:, n_comp:].contiguous().view(B, Hkv, tail, d)
    v_tail = v_all[:, n_comp:].contiguous().view(B, Hkv, tail, d)
    copies = []
    for _ in range(2):
        c = {}
        for name, (k, v, n, qz) in parts.items():
            c[name] = tq.tq_encode(qz, tq.TQ_PROD, k) + tq.tq_encode(qz, tq.TQ_MSE, v)[:2]
        copies.append(c)
    logits = {name: torch.empty((B, Hq, n), dtype=torch.float32, device=dev) for name, (_, _, n, _) in parts.items()}
    ws = {name: torch.empty(tq.scores_workspace_bytes(qz, B, Hq, Hkv, n), dtype=torch.uint8, device=dev)
          for name, (_, _, n, qz) in parts.items()}
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)

    def segments(c):
        return [tq.Segment(parts[nm][3], parts[nm][3], *c[nm][:3], *c[nm][3:5], parts[nm][2]) for nm in ("old", "new")]

    ws_a = torch.empty(tq.attend_segments_workspace_bytes(segments(copies[0]), B, Hq, Hkv, tail), dtype=torch.uint8,
                       device=dev)
    # an aged block: 8 x 4096 tokens of the new segment re-encoded at 2 bits
    na = 4096
    q_old, q_new = parts["old"][3], parts["new"][3]
    age_in = [tq.tq_encode(q_new, tq.TQ_PROD, parts["new"][0][:, :na].contiguous()),
              tq.tq_encode(q_new, tq.TQ_MSE, parts["new"][1][:, :na].contiguous())]
    age_out = [(torch.empty(q_old.code_words(tq.TQ_PROD, nseq, na), dtype=torch.int32, device=dev),
                torch.empty(nseq * na, device=dev), torch.empty(nseq * na, device=dev)),
               (torch.empty(q_old.code_words(tq.TQ_MSE, nseq, na), dtype=torch.int32, device=dev),
                torch.empty(nseq * na, device=dev), None)]
    age_ws = torch.empty(nseq * na * d, dtype=torch.float32, device=dev)
    timer = Timer(torch)

    def step(i, timed):
        w, r = copies[i % 2], copies[(i + 1) % 2]
        e = [timer.mark()]
        for name, (k, v, n, qz) in parts.items():
            tq.tq_encode(qz, tq.TQ_PROD, k, out=w[name][:3])
            tq.tq_encode(qz, tq.TQ_MSE, v, out=(w[name][3], w[name][4], None))
        e.append(timer.mark())
        for name, (k, v, n, qz) in parts.items():
            tq.tq_query_prep(qz, q, Hkv, workspace=ws[name])
            tq.tq_scores_from_prep(qz, B, Hq, Hkv, *r[name][:3], n, ws[name], out=logits[name])
        e.append(timer.mark())
        tq.tq_attend_decode_segments(segments(r), q, Hkv, k_tail, v_tail, out=out, workspace=ws_a)
        e.append(timer.mark())
        tq.tq_requantize(q_new, q_old, tq.TQ_PROD, *age_in[0], nseq, na, out=age_out[0], workspace=age_ws)
        tq.tq_requantize(q_new, q_old, tq.TQ_MSE, age_in[1][0], age_in[1][1], None, nseq, na, out=age_out[1],
                         workspace=age_ws)
        e.append(timer.mark())
        if timed:
            for nm, a, b in zip(("encode", "scores", "attend", "requantize"), e[:-1], e[1:]):
                timer.span(nm, a, b)

    el = _timed_loop(args, torch, step)
    timer.collect()
    rk = {b: 4 * 4 * b + 8 for b in (b_old, b_new)}        # prod key record bytes, d = 128
    rv = {b: (b * d) // 8 + 4 for b in (b_old, b_new)}     # value record bytes
    packed = nseq * (n_old * (rk[b_old] + rv[b_old]) + n_new * (rk[b_new] + rv[b_new]))
    uniform = nseq * n_comp * (rk[b_new] + rv[b_new])
    at = timer.avg_ms("attend")
    at_bytes = packed + nseq * tail * d * 2 * 2
    res = _common(args, el * 1e3 / args.steps,
                  {"workload": f"long-context decay b1 kv8 q32 n131072: {n_old} tokens at {b_old}-bit, {n_new} at "
                               f"{b_new}-bit, 256 bf16 tail"},
                  round(at_bytes / (at * 1e-3) / 1e9, 1), "GB/s",
                  metric="decode attention over a decayed cache, GB/s of packed K+V")
    res["kernels_ms"] = {k2: round(timer.avg_ms(k2), 4) for k2 in timer.acc}
    res["packed_bytes"] = packed
    res["packed_bytes_uniform_4bit"] = uniform
    res["memory_saving_vs_uniform"] = round(1 - packed / uniform, 4)
    res["requantize_tokens_per_s"] = round(2 * nseq * na / (timer.avg_ms("requantize") * 1e-3), 0)
    res["roofline"] = {"kernel": "tq_attend_decode_segments (all its launches)", "bound": "hbm",
                       "achieved": round(at_bytes / (at * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                       "frac": round(at_bytes / (at * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "traffic": None,
                       "algorithmic_bytes_per_launch": at_bytes}
    return res


def cpu_baseline_all():
    """The oracle on a bounded sample of every workload (inputs from the same
    generators at reduced sizes, so the value laws are the workloads'):
    encode throughput (keys/s) and logits throughput (packed key bytes/s and
    query-key pairs/s), all host threads and one thread."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import tq_oracle as o
    from vector_quantization_tq_amd import workloads as W
    cases = []
    wl = W.tiny()
    cases.append(("tiny 4096x128 fp32, 3-bit, 16 queries", 128, 3, wl.arrays["x"].astype(np.float64),
                  wl.arrays["q"].astype(np.float64)))
    wl = W.decode_layer(3, heads=1)
    cases.append(("decode layer (1 head of 32), 8192 keys d128 3-bit, 1 query", 128, 3,
                  wl.arrays["k"][0].astype(np.float64), wl.arrays["q"][:1].astype(np.float64)))
    wl = W.gqa_layer(B=1, Hkv=1, Hq=4, N=16384)
    cases.append(("GQA layer (1 of 64 groups), 16384 keys d128 3-bit, 4 queries", 128, 3,
                  wl.arrays["k"].reshape(-1, 128).astype(np.float64), wl.arrays["q"][0].astype(np.float64)))
    wl = W.long_context(B=1, Hkv=1, Hq=4, N=16384, tail=0)
    cases.append(("long context (1 of 8 groups), 16384 keys d128 4-bit, 4 queries", 128, 4,
                  wl.arrays["k"].reshape(-1, 128).astype(np.float64), wl.arrays["q"][0].astype(np.float64)))
    wl = W.vector_search(4, n=20000, nq=1000)
    cases.append(("vector search, 20000 of 10^6 keys d200 4-bit, 1000 queries", 200, 4,
                  wl.arrays["x"].astype(np.float64), wl.arrays["q"].astype(np.float64)))
    all_threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    for name, d, bits, x, q in cases:
        oq = o.Quantizer(d, bits, 0)
        packed = x.shape[0] * o.record_bytes("prod", d, bits)
        for threads in (all_threads, 1):
            with threadpool_limits(limits=threads):
                t0 = time.perf_counter()
                reps = 0
                while True:
                    idx, b01, nrm, gam = o.encode_prod(oq, x)
                    reps += 1
                    if time.perf_counter() - t0 > 2.0:
                        break
                enc = reps * x.shape[0] / (time.perf_counter() - t0)
                t0 = time.perf_counter()
                reps = 0
                while True:
                    o.scores(oq, q, idx, b01, nrm, gam)
                    reps += 1
                    if time.perf_counter() - t0 > 2.0:
                        break
                el = time.perf_counter() - t0
            print(json.dumps({"workload": name, "threads": threads, "kind": "oracle (float64 numpy)",
                              "encode_keys_per_s": round(enc, 1),
                              "logits_packed_gb_per_s": round(packed * reps / el / 1e9, 4),
                              "logits_pairs_per_s": round(q.shape[0] * x.shape[0] * reps / el, 1)}), flush=True)


def main():
    args = parse()
    if args.cpu_baseline_all:
        cpu_baseline_all()
        return
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only (asked for --gpus {args.gpus}); sharding the path over several GPUs "
              "is not implemented.", file=sys.stderr)
        sys.exit(2)
    if args.kv_width is not None:
        w2 = round(2 * args.kv_width)
        if abs(2 * args.kv_width - w2) > 1e-9 or not 3 <= w2 <= 8:
            raise SystemExit("--kv-width must be a multiple of 0.5 in [1.5, 4]")
        args.bits, args.value_bits = (w2 + 1) // 2, w2 // 2
    import torch

    from vector_quantization_tq_amd import tq
    from vector_quantization_tq_amd import workloads as W
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        copy_calibration(torch, dev)
    if args.workload == "gqa":
        bits = args.bits or 3
        hd = args.head_dim
        res, wl = run_gqa(args, torch, dev, tq, lambda: W.gqa_layer(d=hd),
                          f"gqa-decode-layer b8 kv8 q32 n32768 d{hd} {bits}-bit", bits)
        if (not args.no_cpu_baseline and args.key_mode == "prod" and bits == 3 and not args.value_bits
                and args.v_threshold is None and args.rotation == "haar" and hd == 128):
            res["cpu_baseline"] = cpu_baseline_gqa(wl, args.steps)
    elif args.workload == "long":
        bits = args.bits or 4
        hd = args.head_dim
        res, wl = run_gqa(args, torch, dev, tq, lambda: W.long_context(d=hd),
                          f"long-context b1 kv8 q32 n131072 tail256 d{hd} {bits}-bit", bits, n_tail=256)
    elif args.workload == "decode":
        res = run_decode(args, torch, dev, tq, W)
    elif args.workload == "decay":
        res = run_decay(args, torch, dev, tq, W)
    else:
        res = run_search(args, torch, dev, tq, W)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
