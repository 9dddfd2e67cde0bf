"""Oracle for tree-masked verify attention: plain fp64 CPU definition (see tv_oracle.c).

TEST INFRASTRUCTURE.  Only tests/, the package smoke check and the benchmark's
CPU-baseline leg may import this module.  It shares no code with the HIP
library and never imports it.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libtvoracle.so")
_lib = None

ERRORS = {0: "ok", -1: "null pointer", -2: "bad shape", -3: "bad indptr",
          -4: "kv length shorter than draft count (draft slots missing from kv_indices)",
          -5: "mask block is not n_b * L_b bytes (n_b * n_b prefix-visible): wrong mask stride",
          -6: "slot outside the pool", -7: "allocation failed"}


class OracleError(ValueError):
    def __init__(self, code: int):
        super().__init__("oracle precondition violated: %s (%d)" % (ERRORS.get(code, "?"), code))
        self.code = code


class _Args(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("kv", ctypes.c_void_p), ("kv_indices", ctypes.c_void_p),
                ("kv_indptr", ctypes.c_void_p), ("qo_indptr", ctypes.c_void_p),
                ("mask", ctypes.c_void_p), ("mask_indptr", ctypes.c_void_p),
                ("batch", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("total_q", ctypes.c_int64), ("num_slots", ctypes.c_int64),
                ("total_kv", ctypes.c_int64), ("total_mask", ctypes.c_int64),
                ("sm_scale", ctypes.c_float), ("prefix_visible", ctypes.c_int32),
                ("contiguous_prefix", ctypes.c_int32)]


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            from . import build as _b
            _b.build()
        lib = ctypes.CDLL(_SO)
        lib.tvo_check.argtypes = [ctypes.POINTER(_Args)]
        lib.tvo_check.restype = ctypes.c_int
        lib.tvo_attention.argtypes = [ctypes.POINTER(_Args), ctypes.c_void_p, ctypes.c_int64,
                                      ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        lib.tvo_attention.restype = ctypes.c_int
        lib.tvo_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _pack(q, kv, kv_indices, kv_indptr, qo_indptr, mask, mask_indptr, sm_scale, num_heads,
          prefix_visible=False, contiguous_prefix=False):
    keep = [_c(q, np.uint16), _c(kv, np.uint16), _c(kv_indices, np.int32), _c(kv_indptr, np.int32),
            _c(qo_indptr, np.int32), _c(mask, np.uint8), _c(mask_indptr, np.int32)]
    q_, kv_, ki, kp, qp, m, mp = keep
    if q_.ndim != 3 or q_.shape[1] != num_heads or q_.shape[2] != 576:
        raise ValueError("q must be [N, H, 576] bf16 bits")
    if kv_.ndim != 2 or kv_.shape[1] != 576:
        raise ValueError("kv must be [num_slots, 576] bf16 bits")
    a = _Args(q_.ctypes.data, kv_.ctypes.data, ki.ctypes.data, kp.ctypes.data, qp.ctypes.data,
              m.ctypes.data, mp.ctypes.data, len(qp) - 1, num_heads, q_.shape[0], kv_.shape[0],
              ki.size, m.size, float(np.float32(sm_scale)), int(bool(prefix_visible)),
              int(bool(contiguous_prefix)))
    return a, keep


def check(q, kv, kv_indices, kv_indptr, qo_indptr, mask, mask_indptr, sm_scale, num_heads,
          prefix_visible=False, contiguous_prefix=False) -> int:
    a, keep = _pack(q, kv, kv_indices, kv_indptr, qo_indptr, mask, mask_indptr, sm_scale, num_heads,
                    prefix_visible, contiguous_prefix)
    return _load().tvo_check(ctypes.byref(a))


def attention(q, kv, kv_indices, kv_indptr, qo_indptr, mask, mask_indptr, sm_scale, num_heads,
              rows: Optional[Sequence[int]] = None, threads: int = 0, prefix_visible=False,
              contiguous_prefix=False):
    """fp64 outputs.  rows=None -> (out [N, H, 512], lse [N, H]); otherwise row ids
    g = token * H + head -> (out [len(rows), 512], lse [len(rows)]).
    prefix_visible: the mask holds the draft keys only (n_b x n_b per request)
    and every prefix key is visible.  contiguous_prefix: the prefix keys of
    request b are the pool run starting at kv_indices[kv_indptr[b]]."""
    a, keep = _pack(q, kv, kv_indices, kv_indptr, qo_indptr, mask, mask_indptr, sm_scale, num_heads,
                    prefix_visible, contiguous_prefix)
    N = keep[0].shape[0]
    if rows is None:
        nrows, rp = N * num_heads, None
    else:
        rr = np.ascontiguousarray(rows, dtype=np.int64)
        keep.append(rr)
        nrows, rp = rr.size, rr.ctypes.data
    out = np.empty((nrows, 512), dtype=np.float64)
    lse = np.empty(nrows, dtype=np.float64)
    rc = _load().tvo_attention(ctypes.byref(a), rp, nrows, int(threads), out.ctypes.data,
                               lse.ctypes.data)
    if rc != 0:
        raise OracleError(rc)
    if rows is None:
        return out.reshape(N, num_heads, 512), lse.reshape(N, num_heads)
    return out, lse


def run(w, rows=None, threads: int = 0):
    """Oracle on a tv_workload.Workload."""
    return attention(w.q, w.kv, w.kv_indices, w.kv_indptr, w.qo_indptr, w.mask, w.mask_indptr,
                     w.sm_scale, w.num_heads, rows=rows, threads=threads,
                     prefix_visible=getattr(w, "prefix_visible", False),
                     contiguous_prefix=getattr(w, "contiguous_prefix", False))


def check_workload(w) -> int:
    return check(w.q, w.kv, w.kv_indices, w.kv_indptr, w.qo_indptr, w.mask, w.mask_indptr,
                 w.sm_scale, w.num_heads, prefix_visible=getattr(w, "prefix_visible", False),
                 contiguous_prefix=getattr(w, "contiguous_prefix", False))


def max_threads() -> int:
    return int(_load().tvo_max_threads())
