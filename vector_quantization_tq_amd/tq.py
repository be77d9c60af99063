"""Thin ctypes binding of libtq (include/tq.h).

Argument marshalling only: every step of the hot path runs in libtq's HIP
kernels.  torch is used for device memory (outputs and workspaces are torch
tensors) and for the current HIP stream.  If libtq.so is missing or cannot
be loaded, every call raises; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# TQ_LIBRARY names another build of the same library (a variant built with
# `python -m vector_quantization_tq_amd.build --define ... --out DIR`, for A/B
# measurements); by default the in-tree libtq.so
LIB_PATH = os.environ.get("TQ_LIBRARY") or os.path.join(_HERE, "libtq.so")

TQ_OK, TQ_EINVAL, TQ_EUNSUPPORTED, TQ_EHIP, TQ_ENOMEM, TQ_EWORKSPACE = 0, -1, -2, -3, -4, -5
TQ_PROD, TQ_MSE, TQ_MSE_KEYS = 0, 1, 2
TQ_F32, TQ_BF16 = 0, 1
TQ_ROT_HAAR, TQ_ROT_HADAMARD = 0, 1

EXPORTS = [
    "tq_version", "tq_last_error", "tq_host_normals", "tq_host_rotation", "tq_host_rotation_hadamard",
    "tq_host_qjl_matrix", "tq_host_codebook", "tq_make_quantizer", "tq_make_quantizer_ex", "tq_free_quantizer", "tq_quantizer_info", "tq_set_key_mode", "tq_code_words", "tq_encode",
    "tq_decode", "tq_scores_workspace_bytes", "tq_query_prep", "tq_scores_from_prep", "tq_scores",
    "tq_attend_workspace_bytes", "tq_attend_decode", "tq_attend_decode_sparse", "tq_attend_decode_noalloc",
    "tq_attend_segments_workspace_bytes", "tq_attend_decode_segments", "tq_requantize",
]
MAX_SEGMENTS = 16


class _CSegment(ctypes.Structure):
    """struct tq_segment (include/tq.h)."""
    _fields_ = [("kq", ctypes.c_void_p), ("vq", ctypes.c_void_p), ("kcodes", ctypes.c_void_p),
                ("knorms", ctypes.c_void_p), ("kgammas", ctypes.c_void_p), ("vcodes", ctypes.c_void_p),
                ("vnorms", ctypes.c_void_p), ("n", ctypes.c_int64)]

# size of the library's per-device scratch array used by tq_attend_decode_noalloc (include/tq.h)
NOALLOC_SCRATCH_BYTES = 16 << 20


class TQError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libtq error {code}: {msg}")
        self.code = code


_lib = None


def lib() -> ctypes.CDLL:
    """Load libtq.so (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m vector_quantization_tq_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    c_i, c_i64, c_u64, c_p, c_f = ctypes.c_int, ctypes.c_int64, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_float
    dp = ctypes.POINTER(ctypes.c_double)
    sig = {
        "tq_version": (c_i, []),
        "tq_last_error": (ctypes.c_char_p, []),
        "tq_host_normals": (c_i, [c_u64, c_i, c_i64, dp]),
        "tq_host_rotation": (c_i, [c_i, c_u64, dp]),
        "tq_host_rotation_hadamard": (c_i, [c_i, c_u64, dp]),
        "tq_host_qjl_matrix": (c_i, [c_i, c_i, c_u64, dp]),
        "tq_host_codebook": (c_i, [c_i, c_i, dp, dp]),
        "tq_make_quantizer": (c_p, [c_i, c_i, c_u64]),
        "tq_make_quantizer_ex": (c_p, [c_i, c_i, c_u64, c_i]),
        "tq_free_quantizer": (None, [c_p]),
        "tq_quantizer_info": (c_i, [c_p, ctypes.POINTER(c_i), ctypes.POINTER(c_i), ctypes.POINTER(c_i)]),
        "tq_set_key_mode": (c_i, [c_p, c_i]),
        "tq_code_words": (c_i64, [c_p, c_i, c_i64, c_i64]),
        "tq_encode": (c_i, [c_p, c_i, c_p, c_i, c_i64, c_i64, c_p, c_p, c_p, c_p]),
        "tq_decode": (c_i, [c_p, c_i, c_p, c_p, c_p, c_i64, c_i64, c_p, c_p]),
        "tq_scores_workspace_bytes": (c_i64, [c_p, c_i, c_i, c_i, c_i64, c_i]),
        "tq_scores": (c_i, [c_p, c_p, c_i, c_i, c_i, c_i, c_p, c_p, c_p, c_i64, c_i, c_p, c_p, c_p, c_i64, c_p]),
        "tq_query_prep": (c_i, [c_p, c_p, c_i, c_i, c_i, c_i, c_p, c_i64, c_p]),
        "tq_scores_from_prep": (c_i, [c_p, c_i, c_i, c_i, c_p, c_p, c_p, c_i64, c_p, c_p, c_i64, c_p]),
        "tq_attend_workspace_bytes": (c_i64, [c_p, c_p, c_i, c_i, c_i, c_i64, c_i]),
        "tq_attend_decode": (c_i, [c_p, c_p, c_p, c_i, c_i, c_i, c_i, c_p, c_p, c_p, c_p, c_p, c_i64, c_p, c_p, c_i,
                                   c_f, c_p, c_p, c_i64, c_p]),
        "tq_attend_decode_sparse": (c_i, [c_p, c_p, c_p, c_i, c_i, c_i, c_i, c_p, c_p, c_p, c_p, c_p, c_i64, c_p, c_p,
                                          c_i, c_f, c_f, c_p, c_p, c_i64, c_p]),
        "tq_attend_decode_noalloc": (c_i, [c_p, c_p, c_p, c_i, c_i, c_i, c_i, c_p, c_p, c_p, c_p, c_p, c_i64, c_p, c_p,
                                           c_i, c_f, c_p, c_p]),
        "tq_attend_segments_workspace_bytes": (c_i64, [ctypes.POINTER(_CSegment), c_i, c_i, c_i, c_i, c_i]),
        "tq_attend_decode_segments": (c_i, [ctypes.POINTER(_CSegment), c_i, c_p, c_i, c_i, c_i, c_i, c_p, c_p, c_i, c_f,
                                            c_p, c_p, c_i64, c_p]),
        "tq_requantize": (c_i, [c_p, c_p, c_i, c_p, c_p, c_p, c_i64, c_i64, c_p, c_p, c_p, c_p, c_i64, c_p]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def _check(code: int):
    if code != TQ_OK:
        raise TQError(code, lib().tq_last_error().decode())


def _dptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


# ---------------------------------------------------------------------------
# host-only precompute
# ---------------------------------------------------------------------------
def tq_host_normals(seed: int, tag: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    _check(lib().tq_host_normals(seed, tag, n, _dptr(out)))
    return out


def tq_host_rotation(d: int, seed: int) -> np.ndarray:
    out = np.empty((d, d), dtype=np.float64)
    _check(lib().tq_host_rotation(d, seed, _dptr(out)))
    return out


def tq_host_rotation_hadamard(d: int, seed: int) -> np.ndarray:
    out = np.empty((d, d), dtype=np.float64)
    _check(lib().tq_host_rotation_hadamard(d, seed, _dptr(out)))
    return out


def tq_host_qjl_matrix(m: int, d: int, seed: int) -> np.ndarray:
    out = np.empty((m, d), dtype=np.float64)
    _check(lib().tq_host_qjl_matrix(m, d, seed, _dptr(out)))
    return out


def tq_host_codebook(d: int, levels: int):
    c = np.empty(levels, dtype=np.float64)
    t = np.empty(max(levels - 1, 1), dtype=np.float64)
    _check(lib().tq_host_codebook(d, levels, _dptr(c), _dptr(t)))
    return c, t[:levels - 1]


# ---------------------------------------------------------------------------
# device calls (torch tensors in, torch tensors out)
# ---------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _stream():
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.float32:
        return TQ_F32
    if t.dtype == torch.bfloat16:
        return TQ_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _need_cuda(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("tensors must be contiguous device tensors")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"tensors on different devices ({dev} and {t.device})")


def _need_buf(t, name: str, numel: int, dtypes):
    """The C ABI takes no buffer lengths: a tensor forwarded to it must hold
    at least `numel` elements of one of `dtypes`, or the kernels would read or
    write past its end."""
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}; expected {' or '.join(str(x) for x in dtypes)}")
    if t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements; {numel} needed")


def _codes_dtypes():
    torch = _torch()
    return (torch.int32, torch.uint32) if hasattr(torch, "uint32") else (torch.int32,)


def _check_queries(qz, q, name="queries"):
    torch = _torch()
    if q.dim() != 3:
        raise ValueError(f"{name} must be [B, Hq, d], got shape {tuple(q.shape)}")
    if q.shape[2] != qz.d:
        raise ValueError(f"{name} have d = {q.shape[2]}, the quantizer d = {qz.d}")
    if q.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"{name} must be float32 or bfloat16")


def _check_key_cache(qz, codes, norms, gammas, nseq: int, n: int, prefix=""):
    torch = _torch()
    _need_buf(codes, prefix + "codes", qz.code_words(qz.key_mode, nseq, n), _codes_dtypes())
    _need_buf(norms, prefix + "norms", nseq * n, (torch.float32,))
    if qz.key_mode == TQ_PROD:
        _need_buf(gammas, prefix + "gammas", nseq * n, (torch.float32,))


class Quantizer:
    """Handle of a tq_quantizer (owns the device tables)."""

    def __init__(self, d: int, bits: int, seed: int = 0, rotation: int = TQ_ROT_HAAR):
        L = lib()
        h = L.tq_make_quantizer_ex(d, bits, seed, rotation)
        if not h:
            raise TQError(TQ_EINVAL, L.tq_last_error().decode())
        self._h = ctypes.c_void_p(h)
        dd, bb, mm = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
        _check(L.tq_quantizer_info(self._h, ctypes.byref(dd), ctypes.byref(bb), ctypes.byref(mm)))
        self.d, self.bits, self.m, self.seed, self.rotation = dd.value, bb.value, mm.value, seed, rotation
        self.key_mode = TQ_PROD

    def set_key_mode(self, key_mode: int):
        """TQ_PROD or TQ_MSE_KEYS: the key encoding the scoring calls read."""
        _check(lib().tq_set_key_mode(self._h, key_mode))
        self.key_mode = key_mode

    @property
    def handle(self):
        return self._h

    def close(self):
        if getattr(self, "_h", None):
            lib().tq_free_quantizer(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def code_words(self, mode: int, nseq: int, n: int) -> int:
        w = lib().tq_code_words(self._h, mode, nseq, n)
        if w < 0:
            _check(TQ_EINVAL)
        return w


def tq_make_quantizer(d: int, bits: int, seed: int = 0, rotation: int = TQ_ROT_HAAR) -> Quantizer:
    return Quantizer(d, bits, seed, rotation)


def tq_encode(qz: Quantizer, mode: int, x, out=None):
    """x: [nseq, n, d] or [n, d] float32/bfloat16 device tensor.
    Returns (codes uint32-as-int32 [words], norms [nseq*n], gammas or None)."""
    torch = _torch()
    _need_cuda(x)
    if x.dim() == 2:
        nseq, n = 1, x.shape[0]
    elif x.dim() == 3:
        nseq, n = x.shape[0], x.shape[1]
    else:
        raise ValueError(f"x must be [n, d] or [nseq, n, d], got shape {tuple(x.shape)}")
    if x.shape[-1] != qz.d:
        raise ValueError("last dimension must be d")
    dev = x.device
    if out is None:
        codes = torch.empty(max(qz.code_words(mode, nseq, n), 4), dtype=torch.int32, device=dev)
        norms = torch.empty(max(nseq * n, 4), dtype=torch.float32, device=dev)
        gammas = torch.empty(max(nseq * n, 4), dtype=torch.float32, device=dev) if mode == TQ_PROD else None
    else:
        codes, norms, gammas = out
        _need_cuda(x, codes, norms, gammas)
        _need_buf(codes, "codes", qz.code_words(mode, nseq, n), _codes_dtypes())
        _need_buf(norms, "norms", nseq * n, (torch.float32,))
        if mode == TQ_PROD:
            _need_buf(gammas, "gammas", nseq * n, (torch.float32,))
    _check(lib().tq_encode(qz.handle, mode, _ptr(x), _dtype_code(x), nseq, n, _ptr(codes), _ptr(norms),
                           _ptr(gammas), _stream()))
    return codes, norms, gammas


def tq_decode(qz: Quantizer, mode: int, codes, norms, gammas, nseq: int, n: int, out=None):
    torch = _torch()
    _need_cuda(codes, norms, gammas, out)
    _need_buf(codes, "codes", qz.code_words(mode, nseq, n), _codes_dtypes())
    _need_buf(norms, "norms", nseq * n, (torch.float32,))
    if mode == TQ_PROD:
        _need_buf(gammas, "gammas", nseq * n, (torch.float32,))
    if out is None:
        out = torch.empty((nseq, n, qz.d), dtype=torch.float32, device=codes.device)
    _need_buf(out, "out", nseq * n * qz.d, (torch.float32,))
    _check(lib().tq_decode(qz.handle, mode, _ptr(codes), _ptr(norms), _ptr(gammas), nseq, n, _ptr(out), _stream()))
    return out


def scores_workspace_bytes(qz: Quantizer, B: int, Hq: int, Hkv: int, n: int, topk: int = 0) -> int:
    w = lib().tq_scores_workspace_bytes(qz.handle, B, Hq, Hkv, n, topk)
    if w < 0:
        _check(TQ_EINVAL)
    return w


def tq_scores(qz: Quantizer, q, codes, norms, gammas, Hkv: int, n: int, topk: int = 0, out=None, out_idx=None,
              workspace=None):
    """q: [B, Hq, d] device tensor (float32/bfloat16).  topk == 0 -> logits
    [B, Hq, n]; topk > 0 -> (scores [B, Hq, topk], int64 indices)."""
    torch = _torch()
    _need_cuda(q, codes, norms, gammas, out, out_idx, workspace)
    _check_queries(qz, q)
    B, Hq = q.shape[0], q.shape[1]
    if Hkv < 1 or Hq % Hkv:
        raise ValueError(f"Hq ({Hq}) must be a multiple of Hkv ({Hkv})")
    _check_key_cache(qz, codes, norms, gammas, B * Hkv, n)
    dev = q.device
    if out is None:
        out = torch.empty((B, Hq, topk if topk else n), dtype=torch.float32, device=dev)
    _need_buf(out, "out", B * Hq * (topk if topk else n), (torch.float32,))
    if topk and out_idx is None:
        out_idx = torch.empty((B, Hq, topk), dtype=torch.int64, device=dev)
    if topk:
        _need_buf(out_idx, "out_idx", B * Hq * topk, (torch.int64,))
    if workspace is None:
        workspace = torch.empty(max(scores_workspace_bytes(qz, B, Hq, Hkv, n, topk), 256), dtype=torch.uint8,
                                device=dev)
    _need_buf(workspace, "workspace", scores_workspace_bytes(qz, B, Hq, Hkv, n, topk), (torch.uint8,))
    _check(lib().tq_scores(qz.handle, _ptr(q), _dtype_code(q), B, Hq, Hkv, _ptr(codes), _ptr(norms), _ptr(gammas), n,
                           topk, _ptr(out), _ptr(out_idx) if topk else None, _ptr(workspace), workspace.numel(),
                           _stream()))
    return (out, out_idx) if topk else out


def tq_query_prep(qz: Quantizer, q, Hkv: int, workspace=None):
    """Rotate/project the queries [B, Hq, d] once; returns the workspace."""
    torch = _torch()
    _need_cuda(q, workspace)
    _check_queries(qz, q)
    B, Hq = q.shape[0], q.shape[1]
    if workspace is None:
        workspace = torch.empty(max(scores_workspace_bytes(qz, B, Hq, Hkv, 1, 0), 256), dtype=torch.uint8,
                                device=q.device)
    _need_buf(workspace, "workspace", scores_workspace_bytes(qz, B, Hq, Hkv, 1, 0), (torch.uint8,))
    _check(lib().tq_query_prep(qz.handle, _ptr(q), _dtype_code(q), B, Hq, Hkv, _ptr(workspace), workspace.numel(),
                               _stream()))
    return workspace


def tq_scores_from_prep(qz: Quantizer, B: int, Hq: int, Hkv: int, codes, norms, gammas, n: int, workspace, out=None):
    torch = _torch()
    _need_cuda(codes, norms, gammas, workspace, out)
    if Hkv < 1 or Hq % Hkv:
        raise ValueError(f"Hq ({Hq}) must be a multiple of Hkv ({Hkv})")
    _check_key_cache(qz, codes, norms, gammas, B * Hkv, n)
    _need_buf(workspace, "workspace", scores_workspace_bytes(qz, B, Hq, Hkv, n, 0), (torch.uint8,))
    if out is None:
        out = torch.empty((B, Hq, n), dtype=torch.float32, device=codes.device)
    _need_buf(out, "out", B * Hq * n, (torch.float32,))
    _check(lib().tq_scores_from_prep(qz.handle, B, Hq, Hkv, _ptr(codes), _ptr(norms), _ptr(gammas), n, _ptr(out),
                                     _ptr(workspace), workspace.numel(), _stream()))
    return out


def attend_workspace_bytes(kq: Quantizer, vq: Quantizer, B: int, Hq: int, Hkv: int, n_comp: int, n_tail: int) -> int:
    w = lib().tq_attend_workspace_bytes(kq.handle, vq.handle, B, Hq, Hkv, n_comp, n_tail)
    if w < 0:
        _check(TQ_EINVAL)
    return w


def _check_attend(kq, vq, q, kcodes, knorms, kgammas, vcodes, vnorms, Hkv, n_comp, k_tail, v_tail, out):
    """Checks every tensor an attention call forwards; returns (B, Hq, d, n_tail, out)."""
    torch = _torch()
    _need_cuda(q, kcodes, knorms, kgammas, vcodes, vnorms, k_tail, v_tail, out)
    _check_queries(kq, q)
    B, Hq, d = q.shape
    if Hkv < 1 or Hq % Hkv:
        raise ValueError(f"Hq ({Hq}) must be a multiple of Hkv ({Hkv})")
    if vq.d != kq.d:
        raise ValueError("key and value quantizers differ in d")
    if (k_tail is None) != (v_tail is None):
        raise ValueError("give both tails or neither")
    n_tail = 0 if k_tail is None else k_tail.shape[2]
    if k_tail is not None:
        if k_tail.dtype != torch.bfloat16 or v_tail.dtype != torch.bfloat16:
            raise TypeError("tails must be bfloat16")
        for name, t in (("k_tail", k_tail), ("v_tail", v_tail)):
            if tuple(t.shape) != (B, Hkv, n_tail, d):
                raise ValueError(f"{name} must be [B, Hkv, n_tail, d] = {(B, Hkv, n_tail, d)}, got {tuple(t.shape)}")
    if n_comp > 0:
        _check_key_cache(kq, kcodes, knorms, kgammas, B * Hkv, n_comp, "k")
        _need_buf(vcodes, "vcodes", vq.code_words(TQ_MSE, B * Hkv, n_comp), _codes_dtypes())
        _need_buf(vnorms, "vnorms", B * Hkv * n_comp, (torch.float32,))
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    _need_buf(out, "out", B * Hq * d, (torch.float32,))
    return B, Hq, d, n_tail, out


def tq_attend_decode(kq: Quantizer, vq: Quantizer, q, kcodes, knorms, kgammas, vcodes, vnorms, Hkv: int,
                     n_comp: int, k_tail=None, v_tail=None, scale: float = 0.0, out=None, workspace=None,
                     v_threshold=None):
    """q: [B, Hq, d]; tails: [B, Hkv, n_tail, d] bfloat16 or None.  Returns [B, Hq, d] float32.
    v_threshold (a float in [0, 1)) calls tq_attend_decode_sparse instead."""
    torch = _torch()
    B, Hq, d, n_tail, out = _check_attend(kq, vq, q, kcodes, knorms, kgammas, vcodes, vnorms, Hkv, n_comp, k_tail,
                                          v_tail, out)
    _need_cuda(q, workspace)
    dev = q.device
    if workspace is None:
        workspace = torch.empty(max(attend_workspace_bytes(kq, vq, B, Hq, Hkv, n_comp, n_tail), 256),
                                dtype=torch.uint8, device=dev)
    _need_buf(workspace, "workspace", attend_workspace_bytes(kq, vq, B, Hq, Hkv, n_comp, n_tail), (torch.uint8,))
    if v_threshold is None:
        _check(lib().tq_attend_decode(kq.handle, vq.handle, _ptr(q), _dtype_code(q), B, Hq, Hkv, _ptr(kcodes),
                                      _ptr(knorms), _ptr(kgammas), _ptr(vcodes), _ptr(vnorms), n_comp, _ptr(k_tail),
                                      _ptr(v_tail), n_tail, scale, _ptr(out), _ptr(workspace), workspace.numel(),
                                      _stream()))
    else:
        _check(lib().tq_attend_decode_sparse(kq.handle, vq.handle, _ptr(q), _dtype_code(q), B, Hq, Hkv,
                                             _ptr(kcodes), _ptr(knorms), _ptr(kgammas), _ptr(vcodes), _ptr(vnorms),
                                             n_comp, _ptr(k_tail), _ptr(v_tail), n_tail, scale, float(v_threshold),
                                             _ptr(out), _ptr(workspace), workspace.numel(), _stream()))
    return out


def tq_attend_decode_noalloc(kq: Quantizer, vq: Quantizer, q, kcodes, knorms, kgammas, vcodes, vnorms, Hkv: int,
                             n_comp: int, k_tail=None, v_tail=None, scale: float = 0.0, out=None):
    """tq_attend_decode without a workspace: the library's per-device scratch
    array (NOALLOC_SCRATCH_BYTES) serves instead and the library allocates
    nothing; shapes that need a larger workspace raise TQError.  Calls that
    overlap on one device race on that scratch.  Pass `out` to allocate
    nothing on the Python side either."""
    B, Hq, d, n_tail, out = _check_attend(kq, vq, q, kcodes, knorms, kgammas, vcodes, vnorms, Hkv, n_comp, k_tail,
                                          v_tail, out)
    _check(lib().tq_attend_decode_noalloc(kq.handle, vq.handle, _ptr(q), _dtype_code(q), B, Hq, Hkv, _ptr(kcodes),
                                          _ptr(knorms), _ptr(kgammas), _ptr(vcodes), _ptr(vnorms), n_comp,
                                          _ptr(k_tail), _ptr(v_tail), n_tail, scale, _ptr(out), _stream()))
    return out


class Segment:
    """One age segment of a compressed cache: its key and value quantizers and
    packed arrays, n tokens per (batch, KV head) sequence."""

    def __init__(self, kq: Quantizer, vq: Quantizer, kcodes, knorms, kgammas, vcodes, vnorms, n: int):
        self.kq, self.vq, self.n = kq, vq, n
        self.kcodes, self.knorms, self.kgammas, self.vcodes, self.vnorms = kcodes, knorms, kgammas, vcodes, vnorms


def _c_segments(segments):
    if not 1 <= len(segments) <= MAX_SEGMENTS:
        raise ValueError(f"1 to {MAX_SEGMENTS} segments")
    arr = (_CSegment * len(segments))()
    for i, g in enumerate(segments):
        arr[i] = _CSegment(g.kq.handle.value, g.vq.handle.value, g.kcodes.data_ptr() if g.n else None,
                           g.knorms.data_ptr() if g.n else None,
                           g.kgammas.data_ptr() if (g.n and g.kgammas is not None) else None,
                           g.vcodes.data_ptr() if g.n else None, g.vnorms.data_ptr() if g.n else None, g.n)
    return arr


def attend_segments_workspace_bytes(segments, B: int, Hq: int, Hkv: int, n_tail: int = 0) -> int:
    w = lib().tq_attend_segments_workspace_bytes(_c_segments(segments), len(segments), B, Hq, Hkv, n_tail)
    if w < 0:
        _check(TQ_EINVAL)
    return w


def tq_attend_decode_segments(segments, q, Hkv: int, k_tail=None, v_tail=None, scale: float = 0.0, out=None,
                              workspace=None):
    """Decode attention over a cache kept in age segments (list of Segment,
    e.g. older tokens at fewer bits) plus an optional bf16 tail, one softmax
    over all of them.  q [B, Hq, d]; tails [B, Hkv, n_tail, d]."""
    torch = _torch()
    if not segments:
        raise ValueError("at least one segment")
    s0 = segments[0]
    tensors = [q, k_tail, v_tail, out, workspace]
    for g in segments:
        tensors += [g.kcodes, g.knorms, g.kgammas, g.vcodes, g.vnorms]
    _need_cuda(*tensors)
    B, Hq, d, n_tail, out = _check_attend(s0.kq, s0.vq, q, None, None, None, None, None, Hkv, 0, k_tail, v_tail, out)
    for i, g in enumerate(segments):
        if g.kq.d != d or g.vq.d != d:
            raise ValueError(f"segment {i}: quantizers differ in d")
        if g.n > 0:
            _check_key_cache(g.kq, g.kcodes, g.knorms, g.kgammas, B * Hkv, g.n, f"segment {i} k")
            _need_buf(g.vcodes, f"segment {i} vcodes", g.vq.code_words(TQ_MSE, B * Hkv, g.n), _codes_dtypes())
            _need_buf(g.vnorms, f"segment {i} vnorms", B * Hkv * g.n, (torch.float32,))
    need = attend_segments_workspace_bytes(segments, B, Hq, Hkv, n_tail)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _need_buf(workspace, "workspace", need, (torch.uint8,))
    _check(lib().tq_attend_decode_segments(_c_segments(segments), len(segments), _ptr(q), _dtype_code(q), B, Hq, Hkv,
                                           _ptr(k_tail), _ptr(v_tail), n_tail, scale, _ptr(out), _ptr(workspace),
                                           workspace.numel(), _stream()))
    return out


def tq_requantize(q_from: Quantizer, q_to: Quantizer, mode: int, codes, norms, gammas, nseq: int, n: int, out=None,
                  workspace=None):
    """Re-encode [nseq][n] vectors coded by q_from with q_to (same d, same
    mode): decode, then encode.  Returns (codes, norms, gammas or None) in
    q_to's layout."""
    torch = _torch()
    _need_cuda(codes, norms, gammas, workspace)
    _need_buf(codes, "codes", q_from.code_words(mode, nseq, n), _codes_dtypes())
    _need_buf(norms, "norms", nseq * n, (torch.float32,))
    if mode == TQ_PROD:
        _need_buf(gammas, "gammas", nseq * n, (torch.float32,))
    if q_to.d != q_from.d:
        raise ValueError("quantizers differ in d")
    dev = codes.device
    if out is None:
        out = (torch.empty(max(q_to.code_words(mode, nseq, n), 4), dtype=torch.int32, device=dev),
               torch.empty(max(nseq * n, 4), dtype=torch.float32, device=dev),
               torch.empty(max(nseq * n, 4), dtype=torch.float32, device=dev) if mode == TQ_PROD else None)
    c2, n2, g2 = out
    _need_cuda(c2, n2, g2)
    _need_buf(c2, "codes out", q_to.code_words(mode, nseq, n), _codes_dtypes())
    _need_buf(n2, "norms out", nseq * n, (torch.float32,))
    if mode == TQ_PROD:
        _need_buf(g2, "gammas out", nseq * n, (torch.float32,))
    if workspace is None:
        workspace = torch.empty(max(nseq * n * q_from.d, 4), dtype=torch.float32, device=dev)
    _need_buf(workspace, "workspace", nseq * n * q_from.d, (torch.float32,))
    _check(lib().tq_requantize(q_from.handle, q_to.handle, mode, _ptr(codes), _ptr(norms), _ptr(gammas), nseq, n,
                               _ptr(c2), _ptr(n2), _ptr(g2), _ptr(workspace), workspace.numel() * 4, _stream()))
    return c2, n2, g2
