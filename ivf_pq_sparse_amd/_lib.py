"""ctypes binding of libpqhsa (include/pqhsa.h).

Argument marshalling only: tensors are checked (device, dtype, size,
contiguity) and passed as raw device pointers together with the current
torch stream.  Every computation runs in the HIP library; if the library is
not built, loading fails with an error instead of falling back to anything.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpqhsa.so")

STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported shape", 3: "buffer too small",
          4: "HIP error"}
NUM_STAGES = 6
VARIANT_DEFAULT, VARIANT_STAGED, VARIANT_DENSE, VARIANT_BARRIER_TEST, VARIANT_KEYS_OUT = 0, 1, 2, 3, 4
STAGE_NAMES = ["tables", "scan", "collect", "select", "attend", "merge"]


class PQHSAError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} (status {status})")
        self.status = status


class Shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "num_q_heads", "num_kv_heads", "head_dim", "page_size", "num_pages",
        "max_pages_per_seq", "num_lists", "pq_m", "pq_ksub", "max_context", "n_sink", "n_recent",
        "budget_bp")] + [("scale", ctypes.c_float), ("exact_only", ctypes.c_int32)]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


class WsLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in (
        "lut", "qc", "keys", "bins", "rows", "n_rows", "partials", "flags")] + [
        (n, ctypes.c_int32) for n in ("n_exact_splits", "n_bg_splits", "n_parts")] + [
        (n, ctypes.c_size_t) for n in ("hist", "hist_bytes", "counters", "counters_bytes",
                                       "total")]


class ReuseLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in ("search", "states", "context", "count", "total")]


class IndexLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in (
        "centroids", "codebooks", "list_off", "codes", "pos", "means", "n_indexed", "dropped")]


EXPORTS = [
    "pqhsa_index_bytes", "pqhsa_upload_workspace_bytes", "pqhsa_workspace_bytes",
    "pqhsa_max_selected", "pqhsa_upload_index", "pqhsa_index_dropped", "pqhsa_decode_step",
    "pqhsa_dense_decode_step", "pqhsa_decode_step_profiled", "pqhsa_workspace_layout",
    "pqhsa_index_layout_of", "pqhsa_status_string", "pqhsa_append_workspace_bytes",
    "pqhsa_append_tokens", "pqhsa_reuse_buffer_bytes", "pqhsa_reuse_workspace_bytes",
    "pqhsa_reuse_layout_of", "pqhsa_reuse_clear", "pqhsa_reuse_decode_step",
    "pqhsa_reuse_decode_step_profiled", "pqhsa_step_flags", "pqhsa_decode_step_noalloc",
]
NOALLOC_SCRATCH_BYTES = 128 * 1024 * 1024

_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libpqhsa.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m ivf_pq_sparse_amd.build` "
            "(or __graft_entry__.build()); there is no fallback path")
    lib = ctypes.CDLL(path)
    P, S, I32, SZ = ctypes.c_void_p, ctypes.POINTER(Shape), ctypes.c_int32, ctypes.c_size_t
    sig = {
        "pqhsa_index_bytes": (SZ, [S]),
        "pqhsa_upload_workspace_bytes": (SZ, [S]),
        "pqhsa_workspace_bytes": (SZ, [S, ctypes.c_int]),
        "pqhsa_max_selected": (I32, [S]),
        "pqhsa_upload_index": (ctypes.c_int, [S, P, P, P, P, P, P, P, P, SZ, P, SZ, P]),
        "pqhsa_index_dropped": (ctypes.c_int, [S, P, ctypes.POINTER(ctypes.c_int64), P]),
        "pqhsa_decode_step": (ctypes.c_int, [S, P, P, P, P, P, P, P, P, P, P, SZ, P]),
        "pqhsa_dense_decode_step": (ctypes.c_int, [S, P, P, P, P, P, P, P, P, SZ, P]),
        "pqhsa_decode_step_noalloc": (ctypes.c_int, [S, P, P, P, P, P, P, P, P, P, P]),
        "pqhsa_decode_step_profiled": (ctypes.c_int,
                                       [S, P, P, P, P, P, P, P, P, P, P, SZ, ctypes.c_int, P,
                                        ctypes.POINTER(ctypes.c_int32), P]),
        "pqhsa_workspace_layout": (ctypes.c_int, [S, ctypes.c_int, ctypes.POINTER(WsLayout)]),
        "pqhsa_step_flags": (ctypes.c_int, [S, P, SZ, ctypes.c_int,
                                            ctypes.POINTER(ctypes.c_uint32), P]),
        "pqhsa_append_workspace_bytes": (SZ, [S]),
        "pqhsa_append_tokens": (ctypes.c_int, [S, P, P, P, P, P, ctypes.c_int32, P, P, P, SZ, P]),
        "pqhsa_index_layout_of": (ctypes.c_int, [S, ctypes.POINTER(IndexLayout)]),
        "pqhsa_reuse_buffer_bytes": (SZ, [S, I32]),
        "pqhsa_reuse_workspace_bytes": (SZ, [S, I32]),
        "pqhsa_reuse_layout_of": (ctypes.c_int, [S, I32, ctypes.POINTER(ReuseLayout)]),
        "pqhsa_reuse_clear": (ctypes.c_int, [S, I32, P, SZ, I32, I32, P]),
        "pqhsa_reuse_decode_step": (ctypes.c_int, [S, I32, ctypes.c_float, P, P, P, P, P, P, P,
                                                   SZ, P, P, P, P, P, SZ, P]),
        "pqhsa_reuse_decode_step_profiled": (ctypes.c_int,
                                             [S, I32, ctypes.c_float, P, P, P, P, P, P, P, SZ,
                                              P, P, P, P, P, SZ, P,
                                              ctypes.POINTER(ctypes.c_int32), P]),
        "pqhsa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    _lib = lib
    return lib


# ------------------------------------------------------------------ helpers
def make_shape(*, batch, num_q_heads, num_kv_heads, num_pages, max_pages_per_seq, max_context,
               num_lists=1, n_sink=0, n_recent=0, budget_bp=0, scale=None, head_dim=128,
               page_size=16, pq_m=16, pq_ksub=256, exact_only=0) -> Shape:
    return Shape(batch, num_q_heads, num_kv_heads, head_dim, page_size, num_pages,
                 max_pages_per_seq, num_lists, pq_m, pq_ksub, max_context, n_sink, n_recent,
                 budget_bp, 1.0 / math.sqrt(head_dim) if scale is None else scale,
                 int(exact_only))


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _ptr(t, name, dtype, numel=None, optional=False):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} has {t.numel()} elements, needs {numel}")
    if t.data_ptr() % 16:
        raise ValueError(f"{name} must be 16-byte aligned (the kernels use 16-byte loads)")
    return ctypes.c_void_p(t.data_ptr())


def _check(fn, status):
    if status != 0:
        raise PQHSAError(fn, status)


def _bf16(t):
    """bf16 tensors travel as uint16 bit patterns; accept either."""
    if t is not None and t.dtype == torch.bfloat16:
        return t.view(torch.int16)
    return t


# ------------------------------------------------------------------ queries
def index_bytes(shape: Shape) -> int:
    return load().pqhsa_index_bytes(ctypes.byref(shape))


def upload_workspace_bytes(shape: Shape) -> int:
    return load().pqhsa_upload_workspace_bytes(ctypes.byref(shape))


def workspace_bytes(shape: Shape, dense: bool = False) -> int:
    return load().pqhsa_workspace_bytes(ctypes.byref(shape), int(bool(dense)))


def max_selected(shape: Shape) -> int:
    return load().pqhsa_max_selected(ctypes.byref(shape))


def workspace_layout(shape: Shape, dense: bool = False) -> WsLayout:
    out = WsLayout()
    _check("pqhsa_workspace_layout",
           load().pqhsa_workspace_layout(ctypes.byref(shape), int(bool(dense)), ctypes.byref(out)))
    return out


def index_layout(shape: Shape) -> IndexLayout:
    out = IndexLayout()
    _check("pqhsa_index_layout_of", load().pqhsa_index_layout_of(ctypes.byref(shape), ctypes.byref(out)))
    return out


def status_string(status: int) -> str:
    return load().pqhsa_status_string(status).decode()


# ------------------------------------------------------------------ entry points
def upload_index(shape: Shape, centroids, codebooks, list_ids, codes, n_indexed, v_cache,
                 block_table, index_buf, workspace, stream=None):
    B, H, L, C = shape.batch, shape.num_kv_heads, shape.num_lists, shape.max_context
    u16 = torch.int16
    _check("pqhsa_upload_index", load().pqhsa_upload_index(
        ctypes.byref(shape),
        _ptr(centroids, "centroids", torch.float32, B * H * L * 128),
        _ptr(codebooks, "codebooks", torch.float32, B * H * 16 * 256 * 8),
        _ptr(list_ids, "list_ids", torch.int32, B * H * C),
        _ptr(codes, "codes", torch.uint8, B * H * C * 16),
        _ptr(n_indexed, "n_indexed", torch.int32, B),
        _ptr(_bf16(v_cache), "v_cache", u16, shape.num_pages * 16 * H * 128),
        _ptr(block_table, "block_table", torch.int32, B * shape.max_pages_per_seq),
        _ptr(index_buf, "index_buf", torch.uint8), index_buf.numel(),
        _ptr(workspace, "workspace", torch.uint8), workspace.numel(),
        _stream(stream)))


def step_flags(shape: Shape, workspace, clear: bool = False, stream=None) -> int:
    """The decode workspace's flags word (bit 0: a fused-step barrier wait ran
    out); with clear=True the workspace's counters, flags and histogram are
    zeroed afterwards.  Synchronises the stream."""
    v = ctypes.c_uint32(0)
    _check("pqhsa_step_flags", load().pqhsa_step_flags(
        ctypes.byref(shape), _ptr(workspace, "workspace", torch.uint8), workspace.numel(),
        int(bool(clear)), ctypes.byref(v), _stream(stream)))
    return v.value


def index_dropped(shape: Shape, index_buf, stream=None) -> int:
    v = ctypes.c_int64(0)
    _check("pqhsa_index_dropped", load().pqhsa_index_dropped(
        ctypes.byref(shape), _ptr(index_buf, "index_buf", torch.uint8), ctypes.byref(v),
        _stream(stream)))
    return v.value


def _step_ptrs(shape, q, k_cache, v_cache, block_table, context_lens, out, lse):
    B, Hq, H = shape.batch, shape.num_q_heads, shape.num_kv_heads
    u16 = torch.int16
    return (_ptr(_bf16(q), "q", u16, B * Hq * 128),
            _ptr(_bf16(k_cache), "k_cache", u16, shape.num_pages * 16 * H * 128),
            _ptr(_bf16(v_cache), "v_cache", u16, shape.num_pages * 16 * H * 128),
            _ptr(block_table, "block_table", torch.int32, B * shape.max_pages_per_seq),
            _ptr(context_lens, "context_lens", torch.int32, B),
            _ptr(out, "out", torch.float32, B * Hq * 128),
            _ptr(lse, "lse", torch.float32, B * Hq, optional=True))


def decode_step(shape: Shape, index_buf, q, k_cache, v_cache, block_table, context_lens, out,
                workspace, selected=None, lse=None, stream=None):
    qp, kp, vp, tp, cp, op, lp = _step_ptrs(shape, q, k_cache, v_cache, block_table,
                                            context_lens, out, lse)
    sp = _ptr(selected, "selected", torch.int32,
              shape.batch * shape.num_kv_heads * max(max_selected(shape), 1), optional=True)
    _check("pqhsa_decode_step", load().pqhsa_decode_step(
        ctypes.byref(shape), _ptr(index_buf, "index_buf", torch.uint8), qp, kp, vp, tp, cp, op,
        sp, lp, _ptr(workspace, "workspace", torch.uint8), workspace.numel(), _stream(stream)))


def decode_step_noalloc(shape: Shape, index_buf, q, k_cache, v_cache, block_table,
                        context_lens, out, selected=None, lse=None, stream=None):
    """pqhsa_decode_step_noalloc: the decode step on the library's fixed
    per-device scratch (no workspace argument)."""
    qp, kp, vp, tp, cp, op, lp = _step_ptrs(shape, q, k_cache, v_cache, block_table,
                                            context_lens, out, lse)
    sp = _ptr(selected, "selected", torch.int32,
              shape.batch * shape.num_kv_heads * max(max_selected(shape), 1), optional=True)
    _check("pqhsa_decode_step_noalloc", load().pqhsa_decode_step_noalloc(
        ctypes.byref(shape), _ptr(index_buf, "index_buf", torch.uint8), qp, kp, vp, tp, cp, op,
        sp, lp, _stream(stream)))


def dense_decode_step(shape: Shape, q, k_cache, v_cache, block_table, context_lens, out,
                      workspace, lse=None, stream=None):
    qp, kp, vp, tp, cp, op, lp = _step_ptrs(shape, q, k_cache, v_cache, block_table,
                                            context_lens, out, lse)
    _check("pqhsa_dense_decode_step", load().pqhsa_dense_decode_step(
        ctypes.byref(shape), qp, kp, vp, tp, cp, op, lp,
        _ptr(workspace, "workspace", torch.uint8), workspace.numel(), _stream(stream)))


def decode_step_profiled(shape: Shape, index_buf, q, k_cache, v_cache, block_table,
                         context_lens, out, workspace, events, variant=VARIANT_DEFAULT,
                         selected=None, lse=None, stream=None) -> int:
    """A decode step (variant: VARIANT_DEFAULT, VARIANT_STAGED or VARIANT_DENSE)
    that times its kernels: events[2i], events[2i+1] take the start and end of
    kernel i.  `events` holds 2 * NUM_STAGES HipEvents.  Returns the number of
    kernels launched."""
    qp, kp, vp, tp, cp, op, lp = _step_ptrs(shape, q, k_cache, v_cache, block_table,
                                            context_lens, out, lse)
    sp = _ptr(selected, "selected", torch.int32, optional=True)
    if len(events) < 2 * NUM_STAGES:
        raise ValueError(f"decode_step_profiled needs {2 * NUM_STAGES} events, got {len(events)}")
    arr = (ctypes.c_void_p * len(events))(*[e.handle for e in events])
    dense = variant == VARIANT_DENSE
    ip = None if dense else _ptr(index_buf, "index_buf", torch.uint8)
    nk = ctypes.c_int32(0)
    _check("pqhsa_decode_step_profiled", load().pqhsa_decode_step_profiled(
        ctypes.byref(shape), ip, qp, kp, vp, tp, cp, op, sp, lp,
        _ptr(workspace, "workspace", torch.uint8), workspace.numel(), int(variant), arr,
        ctypes.byref(nk), _stream(stream)))
    return nk.value


def append_workspace_bytes(shape: Shape) -> int:
    return load().pqhsa_append_workspace_bytes(ctypes.byref(shape))


def append_tokens(shape: Shape, index_buf, k_cache, v_cache, block_table, new_n_indexed,
                  max_new: int, list_ids, codes, workspace, stream=None):
    """pqhsa_append_tokens: encode tokens [n_indexed, new_n_indexed) of each
    sequence into `list_ids`/`codes` (token order) and update the index."""
    B, Hkv, cap = shape.batch, shape.num_kv_heads, shape.max_context
    _check("pqhsa_append_tokens", load().pqhsa_append_tokens(
        ctypes.byref(shape), _ptr(index_buf, "index_buf", torch.uint8),
        _ptr(k_cache, "k_cache", torch.int16), _ptr(v_cache, "v_cache", torch.int16),
        _ptr(block_table, "block_table", torch.int32),
        _ptr(new_n_indexed, "new_n_indexed", torch.int32, B), int(max_new),
        _ptr(list_ids, "list_ids", torch.int32, B * Hkv * cap),
        _ptr(codes, "codes", torch.uint8, B * Hkv * cap * 16),
        _ptr(workspace, "workspace", torch.uint8), workspace.numel(), _stream(stream)))


# ------------------------------------------------------------------ query reuse
REUSE_KERNELS = ("search", "attend", "merge")


def reuse_buffer_bytes(shape: Shape, window: int) -> int:
    return load().pqhsa_reuse_buffer_bytes(ctypes.byref(shape), int(window))


def reuse_workspace_bytes(shape: Shape, window: int) -> int:
    return load().pqhsa_reuse_workspace_bytes(ctypes.byref(shape), int(window))


def reuse_layout(shape: Shape, window: int) -> ReuseLayout:
    out = ReuseLayout()
    _check("pqhsa_reuse_layout_of", load().pqhsa_reuse_layout_of(
        ctypes.byref(shape), int(window), ctypes.byref(out)))
    return out


def reuse_clear(shape: Shape, window: int, reuse_buf, seq_begin: int = 0, seq_end=None,
                stream=None):
    """Empty the query rings of sequences [seq_begin, seq_end)."""
    seq_end = shape.batch if seq_end is None else seq_end
    _check("pqhsa_reuse_clear", load().pqhsa_reuse_clear(
        ctypes.byref(shape), int(window), _ptr(reuse_buf, "reuse_buf", torch.uint8),
        reuse_buf.numel(), int(seq_begin), int(seq_end), _stream(stream)))


def reuse_decode_step(shape: Shape, window: int, max_dist2: float, q, q_search, k_cache,
                      v_cache, block_table, context_lens, reuse_buf, out, workspace, lse=None,
                      reused_slot=None, min_dist2=None, events=None, stream=None) -> int:
    """pqhsa_reuse_decode_step (or its profiled form when `events`, 6
    HipEvents, is given).  Returns the number of kernels launched (3)."""
    qp, kp, vp, tp, cp, op, lp = _step_ptrs(shape, q, k_cache, v_cache, block_table,
                                            context_lens, out, lse)
    BQ = shape.batch * shape.num_q_heads
    args = [ctypes.byref(shape), int(window), float(max_dist2), qp,
            _ptr(_bf16(q_search), "q_search", torch.int16, BQ * 128), kp, vp, tp, cp,
            _ptr(reuse_buf, "reuse_buf", torch.uint8), reuse_buf.numel(), op, lp,
            _ptr(reused_slot, "reused_slot", torch.int32, BQ, optional=True),
            _ptr(min_dist2, "min_dist2", torch.float32, BQ, optional=True),
            _ptr(workspace, "workspace", torch.uint8), workspace.numel()]
    if events is None:
        _check("pqhsa_reuse_decode_step", load().pqhsa_reuse_decode_step(*args, _stream(stream)))
        return len(REUSE_KERNELS)
    if len(events) < 2 * len(REUSE_KERNELS):
        raise ValueError(f"reuse_decode_step needs {2 * len(REUSE_KERNELS)} events")
    arr = (ctypes.c_void_p * len(events))(*[e.handle for e in events])
    nk = ctypes.c_int32(0)
    _check("pqhsa_reuse_decode_step_profiled", load().pqhsa_reuse_decode_step_profiled(
        *args, arr, ctypes.byref(nk), _stream(stream)))
    return nk.value


# ------------------------------------------------------------------ HIP events
_hip = None


def _hiprt():
    global _hip
    if _hip is None:
        _hip = ctypes.CDLL("libamdhip64.so")
        _hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        _hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        _hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        _hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        _hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                             ctypes.c_void_p]
    return _hip


class HipEvent:
    """A raw hipEvent_t, recorded by the library on the caller's stream."""

    def __init__(self):
        h = ctypes.c_void_p()
        if _hiprt().hipEventCreate(ctypes.byref(h)) != 0:
            raise RuntimeError("hipEventCreate failed")
        self.handle = h.value

    def record(self, stream=None):
        if _hiprt().hipEventRecord(ctypes.c_void_p(self.handle), _stream(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def synchronize(self):
        _hiprt().hipEventSynchronize(ctypes.c_void_p(self.handle))

    def elapsed_ms(self, end: "HipEvent") -> float:
        v = ctypes.c_float(0)
        if _hiprt().hipEventElapsedTime(ctypes.byref(v), ctypes.c_void_p(self.handle),
                                        ctypes.c_void_p(end.handle)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return v.value

    def __del__(self):
        try:
            if self.handle and _hip is not None:
                _hip.hipEventDestroy(ctypes.c_void_p(self.handle))
        except Exception:
            pass
