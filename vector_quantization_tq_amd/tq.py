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
LIB_PATH = os.path.join(_HERE, "libtq.so")

TQ_OK, TQ_EINVAL, TQ_EUNSUPPORTED, TQ_EHIP, TQ_ENOMEM, TQ_EWORKSPACE = 0, -1, -2, -3, -4, -5
TQ_PROD, TQ_MSE, TQ_MSE_KEYS = 0, 1, 2
TQ_F32, TQ_BF16 = 0, 1
TQ_ROT_HAAR, TQ_ROT_HADAMARD = 0, 1

EXPORTS = [
    "tq_version", "tq_last_error", "tq_host_normals", "tq_host_rotation", "tq_host_rotation_hadamard",
    "tq_host_qjl_matrix", "tq_host_codebook", "tq_make_quantizer", "tq_make_quantizer_ex", "tq_free_quantizer", "tq_quantizer_info", "tq_set_key_mode", "tq_code_words", "tq_encode",
    "tq_decode", "tq_scores_workspace_bytes", "tq_query_prep", "tq_scores_from_prep", "tq_scores",
    "tq_attend_workspace_bytes", "tq_attend_decode", "tq_attend_decode_sparse",
]


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
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous device tensors")


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
    else:
        nseq, n = x.shape[0], x.shape[1]
    if x.shape[-1] != qz.d:
        raise ValueError("last dimension must be d")
    dev = x.device
    if out is None:
        codes = torch.empty(max(qz.code_words(mode, nseq, n), 4), dtype=torch.int32, device=dev)
        norms = torch.empty(max(nseq * n, 4), dtype=torch.float32, device=dev)
        gammas = torch.empty(max(nseq * n, 4), dtype=torch.float32, device=dev) if mode == TQ_PROD else None
    else:
        codes, norms, gammas = out
    _check(lib().tq_encode(qz.handle, mode, _ptr(x), _dtype_code(x), nseq, n, _ptr(codes), _ptr(norms),
                           _ptr(gammas), _stream()))
    return codes, norms, gammas


def tq_decode(qz: Quantizer, mode: int, codes, norms, gammas, nseq: int, n: int, out=None):
    torch = _torch()
    _need_cuda(codes, norms, gammas)
    if out is None:
        out = torch.empty((nseq, n, qz.d), dtype=torch.float32, device=codes.device)
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
    _need_cuda(q, codes, norms, gammas)
    B, Hq = q.shape[0], q.shape[1]
    dev = q.device
    if out is None:
        out = torch.empty((B, Hq, topk if topk else n), dtype=torch.float32, device=dev)
    if topk and out_idx is None:
        out_idx = torch.empty((B, Hq, topk), dtype=torch.int64, device=dev)
    if workspace is None:
        workspace = torch.empty(max(scores_workspace_bytes(qz, B, Hq, Hkv, n, topk), 256), dtype=torch.uint8,
                                device=dev)
    _check(lib().tq_scores(qz.handle, _ptr(q), _dtype_code(q), B, Hq, Hkv, _ptr(codes), _ptr(norms), _ptr(gammas), n,
                           topk, _ptr(out), _ptr(out_idx) if topk else None, _ptr(workspace), workspace.numel(),
                           _stream()))
    return (out, out_idx) if topk else out


def tq_query_prep(qz: Quantizer, q, Hkv: int, workspace=None):
    """Rotate/project the queries [B, Hq, d] once; returns the workspace."""
    torch = _torch()
    _need_cuda(q)
    B, Hq = q.shape[0], q.shape[1]
    if workspace is None:
        workspace = torch.empty(max(scores_workspace_bytes(qz, B, Hq, Hkv, 1, 0), 256), dtype=torch.uint8,
                                device=q.device)
    _check(lib().tq_query_prep(qz.handle, _ptr(q), _dtype_code(q), B, Hq, Hkv, _ptr(workspace), workspace.numel(),
                               _stream()))
    return workspace


def tq_scores_from_prep(qz: Quantizer, B: int, Hq: int, Hkv: int, codes, norms, gammas, n: int, workspace, out=None):
    torch = _torch()
    _need_cuda(codes, norms, gammas, workspace)
    if out is None:
        out = torch.empty((B, Hq, n), dtype=torch.float32, device=codes.device)
    _check(lib().tq_scores_from_prep(qz.handle, B, Hq, Hkv, _ptr(codes), _ptr(norms), _ptr(gammas), n, _ptr(out),
                                     _ptr(workspace), workspace.numel(), _stream()))
    return out


def attend_workspace_bytes(kq: Quantizer, vq: Quantizer, B: int, Hq: int, Hkv: int, n_comp: int, n_tail: int) -> int:
    w = lib().tq_attend_workspace_bytes(kq.handle, vq.handle, B, Hq, Hkv, n_comp, n_tail)
    if w < 0:
        _check(TQ_EINVAL)
    return w


def tq_attend_decode(kq: Quantizer, vq: Quantizer, q, kcodes, knorms, kgammas, vcodes, vnorms, Hkv: int,
                     n_comp: int, k_tail=None, v_tail=None, scale: float = 0.0, out=None, workspace=None,
                     v_threshold=None):
    """q: [B, Hq, d]; tails: [B, Hkv, n_tail, d] bfloat16 or None.  Returns [B, Hq, d] float32.
    v_threshold (a float in [0, 1)) calls tq_attend_decode_sparse instead."""
    torch = _torch()
    _need_cuda(q, kcodes, knorms, kgammas, vcodes, vnorms, k_tail, v_tail)
    B, Hq, d = q.shape
    n_tail = 0 if k_tail is None else k_tail.shape[2]
    if k_tail is not None and (k_tail.dtype != torch.bfloat16 or v_tail.dtype != torch.bfloat16):
        raise TypeError("tails must be bfloat16")
    dev = q.device
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = torch.empty(max(attend_workspace_bytes(kq, vq, B, Hq, Hkv, n_comp, n_tail), 256),
                                dtype=torch.uint8, device=dev)
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
