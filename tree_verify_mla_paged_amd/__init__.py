"""Python binding of libtreeverify (tree-masked verify attention, MI355X / gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libtreeverify.so, called through its C ABI (include/treeverify.h).
torch is used for device memory and streams; tensors are passed by pointer.
There is no fallback: if the library is missing this module fails to import.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY_PATH = os.path.join(_HERE, "libtreeverify.so")

QK_DIM = 576
V_DIM = 512
OUT_BF16 = 0
OUT_F32 = 1
FLAG_PRECISE_P = 1  # probabilities as a bf16 hi + lo pair in the P.V product
FLAG_PREFIX_VISIBLE = 2  # mask holds the draft keys only (n_b x n_b); prefix keys all visible
FLAG_CONTIGUOUS_PREFIX = 4  # prefix keys are the pool run from kv_indices[kv_indptr[b]]

STATUS = {0: "TV_OK", 1: "TV_ERR_NULL", 2: "TV_ERR_SHAPE", 3: "TV_ERR_WORKSPACE",
          4: "TV_ERR_UNSUPPORTED", 5: "TV_ERR_INPUT", 6: "TV_ERR_LAUNCH", 7: "TV_ERR_HIP"}

EXPORTS = ("tv_get_plan", "tv_workspace_bytes", "tv_verify_attn", "tv_verify_attn_timed",
           "tv_verify_attn_static", "tv_check_inputs", "tv_append_draft",
           "tv_status_str")
STATIC_SCRATCH_BYTES = 64 << 20  # the static scratch array behind tv_verify_attn_static


class Problem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("total_q", ctypes.c_int64), ("max_q_len", ctypes.c_int32),
                ("max_kv_len", ctypes.c_int32), ("num_slots", ctypes.c_int64),
                ("total_kv", ctypes.c_int64), ("total_mask", ctypes.c_int64),
                ("num_splits", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("flags", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class AppendProblem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("max_q_len", ctypes.c_int32),
                ("max_kv_len", ctypes.c_int32), ("flags", ctypes.c_int32),
                ("total_q", ctypes.c_int64), ("num_slots", ctypes.c_int64),
                ("total_prefix", ctypes.c_int64), ("total_kv", ctypes.c_int64),
                ("total_mask", ctypes.c_int64)]


class Plan(ctypes.Structure):
    _fields_ = [("split_keys", ctypes.c_int32), ("max_splits", ctypes.c_int32),
                ("row_blocks", ctypes.c_int32), ("merge", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_int64)]


class TreeVerifyError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__("%s: %s (%s)" % (where, status_str(code), STATUS.get(code, code)))
        self.code = code


# The library and torch must share one HIP runtime.  torch ships its own
# libamdhip64; loading it first makes libtreeverify's libamdhip64 dependency
# resolve to that copy instead of a second runtime whose device pointers and
# streams would not be torch's.
import torch  # noqa: E402,F401

if not os.path.exists(LIBRARY_PATH):
    raise ImportError("libtreeverify.so is not built: run `python tree_verify_mla_paged_amd/build.py` "
                      "(hipcc, gfx950) before using the GPU path")

_lib = ctypes.CDLL(LIBRARY_PATH)
_P = ctypes.POINTER(Problem)
_vp = ctypes.c_void_p
_lib.tv_get_plan.argtypes = [_P, ctypes.POINTER(Plan)]
_lib.tv_get_plan.restype = ctypes.c_int
_lib.tv_workspace_bytes.argtypes = [_P]
_lib.tv_workspace_bytes.restype = ctypes.c_size_t
_lib.tv_verify_attn.argtypes = [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_float, _vp, _vp,
                                _vp, ctypes.c_size_t, _vp]
_lib.tv_verify_attn.restype = ctypes.c_int
_lib.tv_verify_attn_timed.argtypes = [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_float, _vp,
                                      _vp, _vp, ctypes.c_size_t, _vp, _vp, _vp]
_lib.tv_verify_attn_timed.restype = ctypes.c_int
_lib.tv_verify_attn_static.argtypes = [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_float, _vp,
                                       _vp, _vp]
_lib.tv_verify_attn_static.restype = ctypes.c_int
_lib.tv_check_inputs.argtypes = [_P, _vp, _vp, _vp, _vp, _vp, ctypes.POINTER(ctypes.c_int32)]
_lib.tv_check_inputs.restype = ctypes.c_int
_lib.tv_append_draft.argtypes = [ctypes.POINTER(AppendProblem)] + [_vp] * 12
_lib.tv_append_draft.restype = ctypes.c_int
_lib.tv_status_str.argtypes = [ctypes.c_int]
_lib.tv_status_str.restype = ctypes.c_char_p


def lib() -> ctypes.CDLL:
    return _lib


def status_str(code: int) -> str:
    return _lib.tv_status_str(int(code)).decode()


def _ptr(x) -> int:
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def _stream(stream) -> int:
    if stream is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


def make_problem(batch: int, num_heads: int, total_q: int, max_q_len: int, max_kv_len: int,
                 num_slots: int, total_kv: int, total_mask: int, num_splits: int = 0,
                 out_dtype: int = OUT_BF16, flags: int = 0) -> Problem:
    return Problem(batch, num_heads, total_q, max_q_len, max_kv_len, num_slots, total_kv,
                   total_mask, num_splits, out_dtype, flags, 0)


def plan(problem: Problem) -> dict:
    pl = Plan()
    rc = _lib.tv_get_plan(ctypes.byref(problem), ctypes.byref(pl))
    if rc != 0:
        raise TreeVerifyError(rc, "tv_get_plan")
    return {f: getattr(pl, f) for f, _ in Plan._fields_}


def workspace_bytes(problem: Problem) -> int:
    return int(_lib.tv_workspace_bytes(ctypes.byref(problem)))


def _need(name: str, x, elem_bytes, count: int):
    """A tensor argument must be a contiguous device tensor with elements of
    `elem_bytes` bytes (an int or a tuple of allowed sizes) and at least `count`
    of them; raw pointers (ints) and None pass unchecked (the C ABI checks
    NULL).  Metadata only: the data is never read here."""
    if x is None or isinstance(x, int):
        return
    sizes = elem_bytes if isinstance(elem_bytes, tuple) else (elem_bytes,)
    if not x.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not x.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if x.element_size() not in sizes:
        raise ValueError("%s has %d-byte elements, expected %s" % (name, x.element_size(), sizes))
    if x.numel() < count:
        raise ValueError("%s holds %d elements, the problem needs %d" % (name, x.numel(), count))


def _check_verify_args(p: Problem, q, kv_buf, kv_indices, kv_indptr, qo_indptr, mask,
                       mask_indptr, out, lse):
    """The extents tv_verify_attn reads and writes, from the problem's host-side
    bounds (q / out / lse rows, pool rows, index and mask entries)."""
    import torch
    rows = int(p.total_q) * int(p.num_heads)
    _need("q", q, 2, rows * QK_DIM)
    _need("kv_buf", kv_buf, 2, int(p.num_slots) * QK_DIM)
    _need("kv_indices", kv_indices, 4, int(p.total_kv))
    for name, x in (("kv_indptr", kv_indptr), ("qo_indptr", qo_indptr),
                    ("mask_indptr", mask_indptr)):
        _need(name, x, 4, int(p.batch) + 1)
    _need("mask", mask, 1, int(p.total_mask))
    _need("out", out, 4 if p.out_dtype == OUT_F32 else 2, rows * V_DIM)
    _need("lse", lse, 4, rows)
    for name, x, dts in (("q", q, (torch.bfloat16, torch.int16, torch.uint16)),
                         ("kv_buf", kv_buf, (torch.bfloat16, torch.int16, torch.uint16)),
                         ("out", out, (torch.float32,) if p.out_dtype == OUT_F32 else
                          (torch.bfloat16, torch.int16, torch.uint16)),
                         ("lse", lse, (torch.float32,)),
                         ("kv_indices", kv_indices, (torch.int32,)),
                         ("kv_indptr", kv_indptr, (torch.int32,)),
                         ("qo_indptr", qo_indptr, (torch.int32,)),
                         ("mask_indptr", mask_indptr, (torch.int32,)),
                         ("mask", mask, (torch.uint8, torch.int8, torch.bool))):
        if x is not None and not isinstance(x, int) and x.dtype not in dts:
            raise ValueError("%s has dtype %s, expected one of %s" % (name, x.dtype, dts))


def _ws_bytes(workspace, workspace_nbytes):
    if workspace_nbytes is None:
        return 0 if workspace is None or isinstance(workspace, int) else \
            workspace.numel() * workspace.element_size()
    if workspace is not None and not isinstance(workspace, int):
        if not workspace.is_cuda or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous device tensor")
        if workspace.numel() * workspace.element_size() < int(workspace_nbytes):
            raise ValueError("workspace is smaller than the workspace_nbytes passed")
    return int(workspace_nbytes)


def verify_attn(problem: Problem, q, kv_buf, kv_indices, kv_indptr, qo_indptr, mask, mask_indptr,
                sm_scale: float, out, lse, workspace, workspace_nbytes: int = None, stream=None):
    """Enqueue tv_verify_attn on `stream` (default: torch's current stream).
    Tensors are device tensors (or raw device pointers as ints); each tensor's
    dtype, contiguity, device and size are checked against the problem first."""
    _check_verify_args(problem, q, kv_buf, kv_indices, kv_indptr, qo_indptr, mask, mask_indptr,
                       out, lse)
    workspace_nbytes = _ws_bytes(workspace, workspace_nbytes)
    rc = _lib.tv_verify_attn(ctypes.byref(problem), _ptr(q), _ptr(kv_buf), _ptr(kv_indices),
                             _ptr(kv_indptr), _ptr(qo_indptr), _ptr(mask), _ptr(mask_indptr),
                             float(sm_scale), _ptr(out), _ptr(lse), _ptr(workspace),
                             int(workspace_nbytes), _stream(stream))
    if rc != 0:
        raise TreeVerifyError(rc, "tv_verify_attn")


def verify_attn_timed(problem: Problem, q, kv_buf, kv_indices, kv_indptr, qo_indptr, mask,
                      mask_indptr, sm_scale: float, out, lse, workspace, workspace_nbytes: int,
                      split_start_event: int, split_stop_event: int, stream=None):
    """tv_verify_attn_timed: events (raw hipEvent_t handles) bracket the split kernel."""
    _check_verify_args(problem, q, kv_buf, kv_indices, kv_indptr, qo_indptr, mask, mask_indptr,
                       out, lse)
    workspace_nbytes = _ws_bytes(workspace, workspace_nbytes)
    rc = _lib.tv_verify_attn_timed(ctypes.byref(problem), _ptr(q), _ptr(kv_buf), _ptr(kv_indices),
                                   _ptr(kv_indptr), _ptr(qo_indptr), _ptr(mask), _ptr(mask_indptr),
                                   float(sm_scale), _ptr(out), _ptr(lse), _ptr(workspace),
                                   int(workspace_nbytes), int(split_start_event),
                                   int(split_stop_event), _stream(stream))
    if rc != 0:
        raise TreeVerifyError(rc, "tv_verify_attn_timed")


def verify_attn_static(problem: Problem, q, kv_buf, kv_indices, kv_indptr, qo_indptr, mask,
                       mask_indptr, sm_scale: float, out, lse, stream=None):
    """Enqueue tv_verify_attn_static: no workspace argument, the library's
    static device scratch (STATIC_SCRATCH_BYTES per GPU) instead.  Calls that
    overlap on one GPU race."""
    _check_verify_args(problem, q, kv_buf, kv_indices, kv_indptr, qo_indptr, mask, mask_indptr,
                       out, lse)
    rc = _lib.tv_verify_attn_static(ctypes.byref(problem), _ptr(q), _ptr(kv_buf),
                                    _ptr(kv_indices), _ptr(kv_indptr), _ptr(qo_indptr),
                                    _ptr(mask), _ptr(mask_indptr), float(sm_scale), _ptr(out),
                                    _ptr(lse), _stream(stream))
    if rc != 0:
        raise TreeVerifyError(rc, "tv_verify_attn_static")


def verify_attn_static_status(problem: Problem, q, kv_buf, kv_indices, kv_indptr, qo_indptr,
                              mask, mask_indptr, sm_scale: float, out, lse,
                              stream: int = 0) -> int:
    """tv_verify_attn_static returning the raw status code (argument-checking tests)."""
    return int(_lib.tv_verify_attn_static(ctypes.byref(problem), _ptr(q), _ptr(kv_buf),
                                          _ptr(kv_indices), _ptr(kv_indptr), _ptr(qo_indptr),
                                          _ptr(mask), _ptr(mask_indptr), float(sm_scale),
                                          _ptr(out), _ptr(lse), int(stream)))


def verify_attn_status(problem: Problem, q, kv_buf, kv_indices, kv_indptr, qo_indptr, mask,
                       mask_indptr, sm_scale: float, out, lse, workspace, workspace_nbytes: int,
                       stream: int = 0) -> int:
    """Same call, returning the raw status code (for argument-checking tests)."""
    return int(_lib.tv_verify_attn(ctypes.byref(problem), _ptr(q), _ptr(kv_buf), _ptr(kv_indices),
                                   _ptr(kv_indptr), _ptr(qo_indptr), _ptr(mask), _ptr(mask_indptr),
                                   float(sm_scale), _ptr(out), _ptr(lse), _ptr(workspace),
                                   int(workspace_nbytes), int(stream)))


def check_inputs(problem: Problem, kv_indices, kv_indptr, qo_indptr, mask_indptr, stream=None):
    """Run tv_check_inputs; returns (status, first bad request or -1)."""
    bad = ctypes.c_int32(-1)
    rc = _lib.tv_check_inputs(ctypes.byref(problem), _ptr(kv_indices), _ptr(kv_indptr),
                              _ptr(qo_indptr), _ptr(mask_indptr), _stream(stream),
                              ctypes.byref(bad))
    return int(rc), int(bad.value)


def make_append_problem(batch: int, max_q_len: int, max_kv_len: int, total_q: int,
                        num_slots: int, total_prefix: int, total_kv: int, total_mask: int,
                        flags: int = 0) -> AppendProblem:
    return AppendProblem(batch, max_q_len, max_kv_len, flags, total_q, num_slots, total_prefix,
                         total_kv, total_mask)


def append_draft_status(problem: AppendProblem, draft_kv, out_cache_loc, prefix_indices,
                        prefix_indptr, qo_indptr, parents, kv_buf, kv_indices, kv_indptr, mask,
                        mask_indptr, stream=None) -> int:
    """tv_append_draft, returning the raw status code."""
    return int(_lib.tv_append_draft(ctypes.byref(problem), _ptr(draft_kv), _ptr(out_cache_loc),
                                    _ptr(prefix_indices), _ptr(prefix_indptr), _ptr(qo_indptr),
                                    _ptr(parents), _ptr(kv_buf), _ptr(kv_indices),
                                    _ptr(kv_indptr), _ptr(mask), _ptr(mask_indptr),
                                    _stream(stream) if stream is not None else 0))


def append_draft(problem: AppendProblem, draft_kv, out_cache_loc, prefix_indices, prefix_indptr,
                 qo_indptr, parents, kv_buf, kv_indices, kv_indptr, mask, mask_indptr,
                 stream=None):
    """Enqueue tv_append_draft on `stream` (default: torch's current stream):
    draft rows into the pool, kv_indices / kv_indptr, and (with parents) the
    tree mask and mask_indptr."""
    rc = _lib.tv_append_draft(ctypes.byref(problem), _ptr(draft_kv), _ptr(out_cache_loc),
                              _ptr(prefix_indices), _ptr(prefix_indptr), _ptr(qo_indptr),
                              _ptr(parents), _ptr(kv_buf), _ptr(kv_indices), _ptr(kv_indptr),
                              _ptr(mask), _ptr(mask_indptr), _stream(stream))
    if rc != 0:
        raise TreeVerifyError(rc, "tv_append_draft")
