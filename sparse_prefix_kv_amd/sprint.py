"""ctypes binding of libsprint.so (C ABI in include/sprint.h).

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, outputs and workspaces are allocated with torch when the caller
does not pass them, and the call runs on torch's current HIP stream.  Every
computation happens in the library's HIP kernels; there is no fallback.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence

import torch  # imported before the library so that both share one HIP runtime

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsprint.so")

F32 = 0
BF16 = 1

_c_void_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_f32 = ctypes.c_float
_f64 = ctypes.c_double
_size = ctypes.c_size_t

_SIGS = {
    "sprint_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "sprint_version": (ctypes.c_int, []),
    "sprint_keep_count": (_i64, [_f64, _i64]),
    "sprint_plan_keep": (ctypes.c_int, [_c_void_p, _c_void_p, _i32, _f64, _f64, _c_void_p,
                                        _c_void_p, _c_void_p]),
    "lmhead_confidence_ws": (_size, [_i64, _i32, _i32, _i32]),
    "lmhead_confidence": (ctypes.c_int, [_c_void_p, _i64, _i32, _c_void_p, _i32, _i32, _c_void_p,
                                         _c_void_p, _c_void_p, _c_void_p, _size, _c_void_p]),
    "lmhead_confidence_unmask_ws": (_size, [_i32, _i32, _i32, _i32, _i32]),
    "lmhead_confidence_unmask": (ctypes.c_int, [_c_void_p, _i32, _i32, _i32, _c_void_p, _i32,
                                                _i32, _c_void_p, _c_void_p, _f32, _i32,
                                                _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                                _size, _c_void_p]),
    "sprint_score_ws": (_size, [_i64, _i32]),
    "sprint_score": (ctypes.c_int, [_c_void_p, _c_void_p, _c_void_p, _i32, _i64, _i32, _i32, _i32,
                                    _f32, _c_void_p, _c_void_p, _c_void_p, _size, _c_void_p]),
    "sprint_prune_kv_ws": (_size, [_i64, _i32]),
    "sprint_prune_kv": (ctypes.c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i32,
                                       _i64, _i64, _c_void_p, _c_void_p, _i32, _i32, _i32,
                                       _c_void_p, _c_void_p, _c_void_p, _c_void_p, _size,
                                       _c_void_p]),
    "block_attend_ws": (_size, [_i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    "block_attend": (ctypes.c_int, [_c_void_p, _i32, _i32, _i32, _c_void_p, _c_void_p, _c_void_p,
                                    _i64, _i32, _c_void_p, _c_void_p, _i32, _i32, _f32, _i32,
                                    _c_void_p, _c_void_p, _size, _c_void_p]),
    "block_attend_noalloc": (ctypes.c_int, [_c_void_p, _i32, _i32, _i32, _c_void_p, _c_void_p,
                                            _c_void_p, _i64, _i32, _c_void_p, _c_void_p, _i32,
                                            _i32, _f32, _i32, _c_void_p, _c_void_p]),
    "unmask_select": (ctypes.c_int, [_c_void_p, _c_void_p, _i32, _i32, _f32, _i32, _c_void_p,
                                     _c_void_p, _c_void_p, _c_void_p]),
    "sprint_score_layers_ws": (_size, [_i64, _i32, _i32]),
    "sprint_score_layers": (ctypes.c_int, [_c_void_p, _i32, _c_void_p, _c_void_p, _i32, _i64, _i32,
                                           _i32, _i32, _f32, _c_void_p, _c_void_p, _c_void_p,
                                           _size, _c_void_p]),
    "sprint_prune_kv_layers": (ctypes.c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                              _c_void_p, _i32, _i64, _i64, _c_void_p, _c_void_p,
                                              _i32, _i32, _i32, _i32, _c_void_p, _c_void_p,
                                              _c_void_p, _c_void_p, _size, _c_void_p]),
    "sprint_score_per_layer": (ctypes.c_int, [_c_void_p, _i32, _c_void_p, _c_void_p, _i32, _i64,
                                              _i32, _i32, _i32, _f32, _c_void_p, _c_void_p,
                                              _c_void_p, _size, _c_void_p]),
    "sprint_prune_kv_per_layer_ws": (_size, [_i64, _i32, _i32]),
    "sprint_prune_kv_per_layer": (ctypes.c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                                 _c_void_p, _i32, _i64, _i64, _c_void_p,
                                                 _c_void_p, _i32, _i32, _i32, _i32, _c_void_p,
                                                 _c_void_p, _c_void_p, _c_void_p, _size,
                                                 _c_void_p]),
    "moe_ffn_ws": (_size, [_i32, _i32, _i32, _i32, _i32]),
    "moe_ffn": (ctypes.c_int, [_c_void_p, _i32, _i32, _c_void_p, _c_void_p, _i32, _i32, _f32,
                               _c_void_p, _c_void_p, _c_void_p, _i32, _i32, _c_void_p,
                               _c_void_p, _c_void_p, _c_void_p, _c_void_p, _size, _c_void_p]),
    "sprint_append_rows": (ctypes.c_int, [_c_void_p, _c_void_p, _i32, _i64, _c_void_p, _i32, _i64,
                                          _c_void_p, _c_void_p, _c_void_p]),
}

EXPORTS = tuple(_SIGS)

_lib = None


class SprintError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {strerror(status)} (status {status})")


def lib() -> ctypes.CDLL:
    """Load libsprint.so once; raise loudly if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               f"`python -m sparse_prefix_kv_amd.build` (hipcc, gfx950)")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(h, name)
            f.restype = res
            f.argtypes = args
        _lib = h
    return _lib


def strerror(status: int) -> str:
    return lib().sprint_strerror(int(status)).decode()


def _check(fn: str, status: int):
    if status != 0:
        raise SprintError(fn, status)


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _dev(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _arg(t, name: str, dtype=None, numel: Optional[int] = None, shape=None):
    """Check a tensor argument's dtype and size (or exact shape), so that a
    wrong buffer raises here instead of being read or written out of range by
    a kernel.  Device and contiguity are checked afterwards, for all
    arguments together (_gpu)."""
    if t is None:
        raise ValueError(f"{name} is required")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and t.shape != shape:
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs {numel}")
    return t


def _gpu(**tensors):
    """Device and contiguity of every tensor argument given (None skipped)."""
    for name, t in tensors.items():
        if t is not None:
            _dev(t, name)


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _ws(size, device, ws: Optional[torch.Tensor]):
    """The caller's workspace, or a new one of size() bytes (the size query
    runs only then: the library checks a given workspace's size itself)."""
    if ws is not None:
        return ws
    return torch.empty(max(int(size()), 256), dtype=torch.uint8, device=device)


# --------------------------------------------------------------------------- host helpers

def sprint_keep_count(r: float, n: int) -> int:
    return int(lib().sprint_keep_count(float(r), int(n)))


def sprint_plan_keep(n_text: Sequence[int], n_img: Sequence[int], r_text: float, r_img: float):
    """Host keep counts -> (keep [nseq*2] int32 list, cu_kept [nseq+1], total_kept)."""
    nseq = len(n_text)
    nt = (ctypes.c_int64 * nseq)(*[int(x) for x in n_text])
    ni = (ctypes.c_int64 * nseq)(*[int(x) for x in n_img])
    keep = (ctypes.c_int32 * (2 * nseq))()
    cu = (ctypes.c_int32 * (nseq + 1))()
    tot = ctypes.c_int64()
    _check("sprint_plan_keep", lib().sprint_plan_keep(
        ctypes.addressof(nt), ctypes.addressof(ni), nseq, float(r_text), float(r_img),
        ctypes.addressof(keep), ctypes.addressof(cu), ctypes.addressof(tot)))
    return list(keep), list(cu), int(tot.value)


# --------------------------------------------------------------------------- workspace queries

def lmhead_confidence_ws(M: int, H: int, V: int, dtype: int) -> int:
    return int(lib().lmhead_confidence_ws(M, H, V, dtype))


def sprint_score_ws(total_L: int, nseq: int) -> int:
    return int(lib().sprint_score_ws(total_L, nseq))


def sprint_prune_kv_ws(total_L: int, nseq: int) -> int:
    return int(lib().sprint_prune_kv_ws(total_L, nseq))


def block_attend_ws(nseq, Lq, Hq, Hkv, D, max_kv, has_block) -> int:
    return int(lib().block_attend_ws(nseq, Lq, Hq, Hkv, D, max_kv, int(bool(has_block))))


# --------------------------------------------------------------------------- device calls

def lmhead_confidence(hidden: torch.Tensor, W: torch.Tensor, conf=None, argmax=None, lse=None,
                      want_lse: bool = False, ws=None, stream=None):
    """Top-1 softmax confidence and argmax of hidden @ W^T.  hidden [M, H], W [V, H]."""
    M, H = hidden.shape
    V = W.shape[0]
    dt = _dt(hidden)
    _arg(hidden, "hidden")
    _arg(W, "W", hidden.dtype, shape=(V, H))
    dev = hidden.device
    f32, i32 = torch.float32, torch.int32
    conf = torch.empty(M, dtype=f32, device=dev) if conf is None else _arg(conf, "conf", f32, M)
    argmax = (torch.empty(M, dtype=i32, device=dev) if argmax is None
              else _arg(argmax, "argmax", i32, M))
    if want_lse and lse is None:
        lse = torch.empty(M, dtype=f32, device=dev)
    if lse is not None:
        _arg(lse, "lse", f32, M)
    _gpu(hidden=hidden, W=W, conf=conf, argmax=argmax, lse=lse)
    ws = _ws(lambda: lmhead_confidence_ws(M, H, V, dt), dev, ws)
    _check("lmhead_confidence", lib().lmhead_confidence(
        _ptr(hidden), M, H, _ptr(W), V, dt, _ptr(conf), _ptr(argmax), _ptr(lse), _ptr(ws),
        ws.numel(), _stream(stream)))
    return (conf, argmax, lse) if want_lse else (conf, argmax)


def sprint_score(K: torch.Tensor, conf: torch.Tensor, cu_len: torch.Tensor, alpha: float = 0.5,
                 ibar=None, score=None, ws=None, stream=None):
    """Mean-normalised key norm and composite score.  K [total_L, Hkv, D]."""
    total_L, Hkv, D = K.shape
    _dt(K)
    _arg(K, "K")
    f32 = torch.float32
    _arg(conf, "conf", f32, total_L)
    _arg(cu_len, "cu_len", torch.int32)
    nseq = cu_len.numel() - 1
    dev = K.device
    ibar = torch.empty(total_L, dtype=f32, device=dev) if ibar is None else _arg(ibar, "ibar", f32, total_L)
    score = (torch.empty(total_L, dtype=f32, device=dev) if score is None
             else _arg(score, "score", f32, total_L))
    _gpu(K=K, conf=conf, cu_len=cu_len, ibar=ibar, score=score)
    ws = _ws(lambda: sprint_score_ws(total_L, nseq), dev, ws)
    _check("sprint_score", lib().sprint_score(
        _ptr(K), _ptr(conf), _ptr(cu_len), nseq, total_L, Hkv, D, _dt(K), float(alpha),
        _ptr(ibar), _ptr(score), _ptr(ws), ws.numel(), _stream(stream)))
    return ibar, score


def sprint_prune_kv(score, modality, cu_len, keep, cu_kept, total_kept: int, K, V,
                    K_out=None, V_out=None, kept_idx=None, ws=None, stream=None):
    """Per-modality top-k selection and compaction into a contiguous pruned cache."""
    total_L, Hkv, D = K.shape
    _dt(K)
    _arg(K, "K")
    _arg(V, "V", K.dtype, shape=K.shape)
    i32 = torch.int32
    _arg(cu_len, "cu_len", i32)
    nseq = cu_len.numel() - 1
    _arg(score, "score", torch.float32, total_L)
    _arg(modality, "modality", torch.uint8, total_L)
    _arg(keep, "keep", i32, 2 * nseq)
    _arg(cu_kept, "cu_kept", i32, nseq + 1)
    if not 0 <= total_kept <= total_L:
        raise ValueError("total_kept must lie in [0, total_L]")
    dev = K.device
    if K_out is None:
        K_out = torch.empty((max(total_kept, 1), Hkv, D), dtype=K.dtype, device=dev)[:total_kept]
    if V_out is None:
        V_out = torch.empty((max(total_kept, 1), Hkv, D), dtype=V.dtype, device=dev)[:total_kept]
    if kept_idx is None:
        kept_idx = torch.empty(max(total_kept, 1), dtype=i32, device=dev)[:total_kept]
    if total_kept:
        _arg(K_out, "K_out", K.dtype, total_kept * Hkv * D)
        _arg(V_out, "V_out", K.dtype, total_kept * Hkv * D)
        _arg(kept_idx, "kept_idx", i32, total_kept)
    _gpu(score=score, modality=modality, cu_len=cu_len, keep=keep, cu_kept=cu_kept, K=K, V=V,
         K_out=K_out, V_out=V_out, kept_idx=kept_idx)
    ws = _ws(lambda: sprint_prune_kv_ws(total_L, nseq), dev, ws)
    _check("sprint_prune_kv", lib().sprint_prune_kv(
        _ptr(score), _ptr(modality), _ptr(cu_len), _ptr(keep), _ptr(cu_kept), nseq, total_L,
        int(total_kept), _ptr(K), _ptr(V), Hkv, D, _dt(K), _ptr(K_out), _ptr(V_out),
        _ptr(kept_idx), _ptr(ws), ws.numel(), _stream(stream)))
    return K_out, V_out, kept_idx


def block_attend(Q, Kp, Vp, cu_kv, max_kv: int, Kb=None, Vb=None, scale: Optional[float] = None,
                 O=None, ws=None, stream=None):
    """softmax(Q K^T * scale) V over [prefix ; block] with GQA.  Q [nseq, Lq, Hq, D]."""
    nseq, Lq, Hq, D = Q.shape
    _dt(Q)
    _arg(Q, "Q")
    total_kv, Hkv = Kp.shape[0], Kp.shape[1]
    _arg(Kp, "Kp", Q.dtype, shape=(total_kv, Hkv, D))
    _arg(Vp, "Vp", Q.dtype, shape=(total_kv, Hkv, D))
    _arg(cu_kv, "cu_kv", torch.int32, shape=(nseq + 1,))
    if (Kb is None) != (Vb is None):
        raise ValueError("Kb and Vb go together")
    if Kb is not None:
        _arg(Kb, "Kb", Q.dtype, shape=(nseq, Lq, Hkv, D))
        _arg(Vb, "Vb", Q.dtype, shape=(nseq, Lq, Hkv, D))
    if scale is None:
        scale = D ** -0.5
    dev = Q.device
    O = torch.empty_like(Q) if O is None else _arg(O, "O", Q.dtype, Q.numel())
    _gpu(Q=Q, Kp=Kp, Vp=Vp, cu_kv=cu_kv, Kb=Kb, Vb=Vb, O=O)
    ws = _ws(lambda: block_attend_ws(nseq, Lq, Hq, Hkv, D, max_kv, Kb is not None), dev, ws)
    _check("block_attend", lib().block_attend(
        _ptr(Q), nseq, Lq, Hq, _ptr(Kp) if total_kv else None, _ptr(Vp) if total_kv else None,
        _ptr(cu_kv), total_kv, int(max_kv), _ptr(Kb), _ptr(Vb), Hkv, D, float(scale), _dt(Q),
        _ptr(O), _ptr(ws), ws.numel(), _stream(stream)))
    return O


def block_attend_noalloc(Q, Kp, Vp, cu_kv, max_kv: int, Kb=None, Vb=None,
                         scale: Optional[float] = None, O=None, stream=None):
    """block_attend with its key-range partials in the library's fixed
    16 MiB device array instead of a workspace (the call allocates no device
    memory; `O` must be given for that).  Calls overlapping on one GPU race."""
    nseq, Lq, Hq, D = Q.shape
    _dt(Q)
    _arg(Q, "Q")
    total_kv, Hkv = Kp.shape[0], Kp.shape[1]
    _arg(Kp, "Kp", Q.dtype, shape=(total_kv, Hkv, D))
    _arg(Vp, "Vp", Q.dtype, shape=(total_kv, Hkv, D))
    _arg(cu_kv, "cu_kv", torch.int32, shape=(nseq + 1,))
    if (Kb is None) != (Vb is None):
        raise ValueError("Kb and Vb go together")
    if Kb is not None:
        _arg(Kb, "Kb", Q.dtype, shape=(nseq, Lq, Hkv, D))
        _arg(Vb, "Vb", Q.dtype, shape=(nseq, Lq, Hkv, D))
    if scale is None:
        scale = D ** -0.5
    O = torch.empty_like(Q) if O is None else _arg(O, "O", Q.dtype, Q.numel())
    _gpu(Q=Q, Kp=Kp, Vp=Vp, cu_kv=cu_kv, Kb=Kb, Vb=Vb, O=O)
    _check("block_attend_noalloc", lib().block_attend_noalloc(
        _ptr(Q), nseq, Lq, Hq, _ptr(Kp) if total_kv else None, _ptr(Vp) if total_kv else None,
        _ptr(cu_kv), total_kv, int(max_kv), _ptr(Kb), _ptr(Vb), Hkv, D, float(scale), _dt(Q),
        _ptr(O), _stream(stream)))
    return O


def unmask_select(conf, argmax, masked, tokens, tau: float, steps_left: int, n_accepted=None,
                  stream=None):
    """One confidence-adaptive unmasking step; updates masked and tokens in place."""
    nseq, Lq = conf.shape
    _arg(conf, "conf", torch.float32)
    _arg(argmax, "argmax", torch.int32, shape=(nseq, Lq))
    _arg(masked, "masked", torch.uint8, shape=(nseq, Lq))
    _arg(tokens, "tokens", torch.int32, shape=(nseq, Lq))
    if n_accepted is None:
        n_accepted = torch.empty(nseq, dtype=torch.int32, device=conf.device)
    _arg(n_accepted, "n_accepted", torch.int32, nseq)
    _gpu(conf=conf, argmax=argmax, masked=masked, tokens=tokens, n_accepted=n_accepted)
    _check("unmask_select", lib().unmask_select(
        _ptr(conf), _ptr(argmax), nseq, Lq, float(tau), int(steps_left), _ptr(masked),
        _ptr(tokens), _ptr(n_accepted), _stream(stream)))
    return n_accepted


def lmhead_confidence_unmask_ws(nseq, Lq, H, V, dtype) -> int:
    return int(lib().lmhead_confidence_unmask_ws(nseq, Lq, H, V, dtype))


def lmhead_confidence_unmask(hidden, W, masked, tokens, tau: float, steps_left: int, conf=None,
                             argmax=None, n_accepted=None, ws=None, stream=None):
    """The block's LM-head confidences, then one unmasking step, in one call.
    hidden [nseq*Lq, H]; masked, tokens [nseq, Lq] (updated in place)."""
    nseq, Lq = masked.shape
    M, H = hidden.shape
    V = W.shape[0]
    dt = _dt(hidden)
    _arg(hidden, "hidden", shape=(nseq * Lq, H))
    _arg(W, "W", hidden.dtype, shape=(V, H))
    _arg(masked, "masked", torch.uint8, shape=(nseq, Lq))
    _arg(tokens, "tokens", torch.int32, shape=(nseq, Lq))
    dev = hidden.device
    f32, i32 = torch.float32, torch.int32
    conf = torch.empty(M, dtype=f32, device=dev) if conf is None else _arg(conf, "conf", f32, M)
    argmax = (torch.empty(M, dtype=i32, device=dev) if argmax is None
              else _arg(argmax, "argmax", i32, M))
    n_accepted = (torch.empty(nseq, dtype=i32, device=dev) if n_accepted is None
                  else _arg(n_accepted, "n_accepted", i32, nseq))
    _gpu(hidden=hidden, W=W, masked=masked, tokens=tokens, conf=conf, argmax=argmax,
         n_accepted=n_accepted)
    ws = _ws(lambda: lmhead_confidence_unmask_ws(nseq, Lq, H, V, dt), dev, ws)
    _check("lmhead_confidence_unmask", lib().lmhead_confidence_unmask(
        _ptr(hidden), nseq, Lq, H, _ptr(W), V, dt, _ptr(conf), _ptr(argmax), float(tau),
        int(steps_left), _ptr(masked), _ptr(tokens), _ptr(n_accepted), _ptr(ws), ws.numel(),
        _stream(stream)))
    return conf, argmax, n_accepted


def sprint_append_rows(old, cu_old, blk, out=None, cu_out=None, stream=None):
    """Append each sequence's block rows after its packed rows (prefix growth).

    old [total_old, ...] packed by cu_old [nseq+1]; blk [nseq, n_blk, ...] or
    [nseq*n_blk, ...] with the same row shape and dtype.  Returns (out, cu_out).
    """
    _arg(old, "old")
    _arg(blk, "blk", old.dtype)
    _arg(cu_old, "cu_old", torch.int32)
    nseq = cu_old.numel() - 1
    row_shape = tuple(old.shape[1:])
    row_elems = math.prod(row_shape)
    total_old = old.shape[0]
    if row_elems == 0 or blk.numel() % (row_elems * nseq) != 0:
        raise ValueError("blk must hold whole rows of old's shape, the same count per sequence")
    n_blk = blk.numel() // (row_elems * nseq)
    row_bytes = old.element_size() * row_elems
    total = total_old + nseq * n_blk
    dev = old.device
    if out is None:
        out = torch.empty((total, *row_shape), dtype=old.dtype, device=dev)
    _arg(out, "out", old.dtype, total * row_elems)
    if cu_out is None:
        cu_out = torch.empty(nseq + 1, dtype=torch.int32, device=dev)
    _arg(cu_out, "cu_out", torch.int32, nseq + 1)
    _gpu(old=old, blk=blk, cu_old=cu_old, out=out, cu_out=cu_out)
    _check("sprint_append_rows", lib().sprint_append_rows(
        _ptr(old) if total_old else None, _ptr(cu_old), nseq, total_old,
        _ptr(blk) if n_blk else None, n_blk, row_bytes, _ptr(out) if total else None,
        _ptr(cu_out), _stream(stream)))
    return out, cu_out


def sprint_score_layers_ws(total_L: int, nseq: int, n_layers: int) -> int:
    return int(lib().sprint_score_layers_ws(total_L, nseq, n_layers))


def sprint_score_layers(K, conf, cu_len, alpha: float = 0.5, ibar=None, score=None, ws=None,
                        stream=None):
    """Layer-mean key-norm importance and composite score.  K [n_layers, total_L, Hkv, D]."""
    n_layers, total_L, Hkv, D = K.shape
    _dt(K)
    _arg(K, "K")
    f32 = torch.float32
    _arg(conf, "conf", f32, total_L)
    _arg(cu_len, "cu_len", torch.int32)
    nseq = cu_len.numel() - 1
    dev = K.device
    ibar = torch.empty(total_L, dtype=f32, device=dev) if ibar is None else _arg(ibar, "ibar", f32, total_L)
    score = (torch.empty(total_L, dtype=f32, device=dev) if score is None
             else _arg(score, "score", f32, total_L))
    _gpu(K=K, conf=conf, cu_len=cu_len, ibar=ibar, score=score)
    ws = _ws(lambda: sprint_score_layers_ws(total_L, nseq, n_layers), dev, ws)
    _check("sprint_score_layers", lib().sprint_score_layers(
        _ptr(K), n_layers, _ptr(conf), _ptr(cu_len), nseq, total_L, Hkv, D, _dt(K),
        float(alpha), _ptr(ibar), _ptr(score), _ptr(ws), ws.numel(), _stream(stream)))
    return ibar, score


def sprint_prune_kv_layers(score, modality, cu_len, keep, cu_kept, total_kept: int, K, V,
                           K_out=None, V_out=None, kept_idx=None, ws=None, stream=None):
    """One kept set compacted in every layer's cache.  K, V [n_layers, total_L, Hkv, D]."""
    n_layers, total_L, Hkv, D = K.shape
    _dt(K)
    _arg(K, "K")
    _arg(V, "V", K.dtype, shape=K.shape)
    i32 = torch.int32
    _arg(cu_len, "cu_len", i32)
    nseq = cu_len.numel() - 1
    _arg(score, "score", torch.float32, total_L)
    _arg(modality, "modality", torch.uint8, total_L)
    _arg(keep, "keep", i32, 2 * nseq)
    _arg(cu_kept, "cu_kept", i32, nseq + 1)
    if not 0 <= total_kept <= total_L:
        raise ValueError("total_kept must lie in [0, total_L]")
    dev = K.device
    shape = (n_layers, max(total_kept, 1), Hkv, D)
    if K_out is None:
        K_out = torch.empty(shape, dtype=K.dtype, device=dev)[:, :total_kept]
    if V_out is None:
        V_out = torch.empty(shape, dtype=V.dtype, device=dev)[:, :total_kept]
    if kept_idx is None:
        kept_idx = torch.empty(max(total_kept, 1), dtype=i32, device=dev)[:total_kept]
    if total_kept:
        _arg(K_out, "K_out", K.dtype, shape=(n_layers, total_kept, Hkv, D))
        _arg(V_out, "V_out", K.dtype, shape=(n_layers, total_kept, Hkv, D))
        _arg(kept_idx, "kept_idx", i32, total_kept)
    _gpu(score=score, modality=modality, cu_len=cu_len, keep=keep, cu_kept=cu_kept, K=K, V=V,
         K_out=K_out, V_out=V_out, kept_idx=kept_idx)
    ws = _ws(lambda: sprint_prune_kv_ws(total_L, nseq), dev, ws)
    _check("sprint_prune_kv_layers", lib().sprint_prune_kv_layers(
        _ptr(score), _ptr(modality), _ptr(cu_len), _ptr(keep), _ptr(cu_kept), nseq, total_L,
        int(total_kept), _ptr(K), _ptr(V), n_layers, Hkv, D, _dt(K), _ptr(K_out), _ptr(V_out),
        _ptr(kept_idx), _ptr(ws), ws.numel(), _stream(stream)))
    return K_out, V_out, kept_idx


def sprint_score_per_layer(K, conf, cu_len, alpha: float = 0.5, ibar=None, score=None, ws=None,
                           stream=None):
    """Each layer's own key-norm importance and score.  K [n_layers, total_L, Hkv, D];
    ibar, score [n_layers, total_L]."""
    n_layers, total_L, Hkv, D = K.shape
    _dt(K)
    _arg(K, "K")
    f32 = torch.float32
    _arg(conf, "conf", f32, total_L)
    _arg(cu_len, "cu_len", torch.int32)
    nseq = cu_len.numel() - 1
    dev = K.device
    shape = (n_layers, total_L)
    ibar = (torch.empty(shape, dtype=f32, device=dev) if ibar is None
            else _arg(ibar, "ibar", f32, shape=shape))
    score = (torch.empty(shape, dtype=f32, device=dev) if score is None
             else _arg(score, "score", f32, shape=shape))
    _gpu(K=K, conf=conf, cu_len=cu_len, ibar=ibar, score=score)
    ws = _ws(lambda: sprint_score_layers_ws(total_L, nseq, n_layers), dev, ws)
    _check("sprint_score_per_layer", lib().sprint_score_per_layer(
        _ptr(K), n_layers, _ptr(conf), _ptr(cu_len), nseq, total_L, Hkv, D, _dt(K),
        float(alpha), _ptr(ibar), _ptr(score), _ptr(ws), ws.numel(), _stream(stream)))
    return ibar, score


def sprint_prune_kv_per_layer_ws(total_L: int, nseq: int, n_layers: int) -> int:
    return int(lib().sprint_prune_kv_per_layer_ws(total_L, nseq, n_layers))


def sprint_prune_kv_per_layer(score, modality, cu_len, keep, cu_kept, total_kept: int, K, V,
                              K_out=None, V_out=None, kept_idx=None, ws=None, stream=None):
    """Each layer's own kept set compacted in its cache.  score [n_layers, total_L];
    K, V [n_layers, total_L, Hkv, D]; kept_idx [n_layers, total_kept]."""
    n_layers, total_L, Hkv, D = K.shape
    _dt(K)
    _arg(K, "K")
    _arg(V, "V", K.dtype, shape=K.shape)
    i32 = torch.int32
    _arg(cu_len, "cu_len", i32)
    nseq = cu_len.numel() - 1
    _arg(score, "score", torch.float32, shape=(n_layers, total_L))
    _arg(modality, "modality", torch.uint8, total_L)
    _arg(keep, "keep", i32, 2 * nseq)
    _arg(cu_kept, "cu_kept", i32, nseq + 1)
    if not 0 <= total_kept <= total_L:
        raise ValueError("total_kept must lie in [0, total_L]")
    dev = K.device
    shape = (n_layers, max(total_kept, 1), Hkv, D)
    if K_out is None:
        K_out = torch.empty(shape, dtype=K.dtype, device=dev)[:, :total_kept]
    if V_out is None:
        V_out = torch.empty(shape, dtype=V.dtype, device=dev)[:, :total_kept]
    if kept_idx is None:
        kept_idx = torch.empty((n_layers, max(total_kept, 1)), dtype=i32, device=dev)[:, :total_kept]
    if total_kept:
        _arg(K_out, "K_out", K.dtype, shape=(n_layers, total_kept, Hkv, D))
        _arg(V_out, "V_out", K.dtype, shape=(n_layers, total_kept, Hkv, D))
        _arg(kept_idx, "kept_idx", i32, shape=(n_layers, total_kept))
    _gpu(score=score, modality=modality, cu_len=cu_len, keep=keep, cu_kept=cu_kept, K=K, V=V,
         K_out=K_out, V_out=V_out, kept_idx=kept_idx)
    ws = _ws(lambda: sprint_prune_kv_per_layer_ws(total_L, nseq, n_layers), dev, ws)
    _check("sprint_prune_kv_per_layer", lib().sprint_prune_kv_per_layer(
        _ptr(score), _ptr(modality), _ptr(cu_len), _ptr(keep), _ptr(cu_kept), nseq, total_L,
        int(total_kept), _ptr(K), _ptr(V), n_layers, Hkv, D, _dt(K), _ptr(K_out), _ptr(V_out),
        _ptr(kept_idx), _ptr(ws), ws.numel(), _stream(stream)))
    return K_out, V_out, kept_idx


def moe_ffn_ws(M: int, H: int, n_experts: int, top_k: int, inter: int) -> int:
    return int(lib().moe_ffn_ws(M, H, n_experts, top_k, inter))


def moe_ffn(x, w_router, bias, w_gate, w_up, w_down, top_k: int, route_scale: float = 2.5,
            residual=None, y=None, expert_ids=None, gates=None, ws=None, stream=None):
    """MoE FFN with sigmoid routing, bias-steered top-k and SwiGLU experts.
    x [M, H]; w_router [E, H]; bias [E] float32; w_gate, w_up [E, I, H];
    w_down [E, H, I].  Returns (y, expert_ids, gates)."""
    M, H = x.shape
    E, inter = w_gate.shape[0], w_gate.shape[1]
    _dt(x)
    _arg(x, "x")
    _arg(w_router, "w_router", x.dtype, shape=(E, H))
    _arg(bias, "bias", torch.float32, shape=(E,))
    _arg(w_gate, "w_gate", x.dtype, shape=(E, inter, H))
    _arg(w_up, "w_up", x.dtype, shape=(E, inter, H))
    _arg(w_down, "w_down", x.dtype, shape=(E, H, inter))
    if residual is not None:
        _arg(residual, "residual", x.dtype, shape=(M, H))
    dev = x.device
    y = torch.empty_like(x) if y is None else _arg(y, "y", x.dtype, shape=(M, H))
    if expert_ids is None:
        expert_ids = torch.empty((M, top_k), dtype=torch.int32, device=dev)
    if gates is None:
        gates = torch.empty((M, top_k), dtype=torch.float32, device=dev)
    _arg(expert_ids, "expert_ids", torch.int32, M * top_k)
    _arg(gates, "gates", torch.float32, M * top_k)
    _gpu(x=x, w_router=w_router, bias=bias, w_gate=w_gate, w_up=w_up, w_down=w_down,
         residual=residual, y=y, expert_ids=expert_ids, gates=gates)
    ws = _ws(lambda: moe_ffn_ws(M, H, E, top_k, inter), dev, ws)
    _check("moe_ffn", lib().moe_ffn(
        _ptr(x), M, H, _ptr(w_router), _ptr(bias), E, top_k, float(route_scale), _ptr(w_gate),
        _ptr(w_up), _ptr(w_down), inter, _dt(x), _ptr(residual), _ptr(y), _ptr(expert_ids),
        _ptr(gates), _ptr(ws), ws.numel(), _stream(stream)))
    return y, expert_ids, gates
