"""PQ-HSA decode attention for AMD Instinct MI355X (gfx950).

Python face of libpqhsa (include/pqhsa.h).  The functions in `_lib` mirror
the C entry points one to one; `PQHSADecoder` owns the index buffer and the
workspaces that those entry points need.  torch supplies device memory and
streams; all computation runs in the HIP kernels.
"""
from __future__ import annotations

import torch

from . import _lib
from ._lib import (  # noqa: F401
    EXPORTS,
    append_tokens,
    append_workspace_bytes,
    NOALLOC_SCRATCH_BYTES,
    NUM_STAGES,
    VARIANT_BARRIER_TEST,
    VARIANT_DEFAULT,
    VARIANT_DENSE,
    VARIANT_KEYS_OUT,
    VARIANT_STAGED,
    STAGE_NAMES,
    HipEvent,
    PQHSAError,
    REUSE_KERNELS,
    ReuseLayout,
    Shape,
    decode_step,
    decode_step_noalloc,
    decode_step_profiled,
    dense_decode_step,
    index_bytes,
    index_dropped,
    index_layout,
    load,
    make_shape,
    max_selected,
    reuse_buffer_bytes,
    reuse_clear,
    reuse_decode_step,
    reuse_layout,
    reuse_workspace_bytes,
    step_flags,
    status_string,
    upload_index,
    upload_workspace_bytes,
    workspace_bytes,
    workspace_layout,
)


class PQHSADecoder:
    """Owns one index buffer and the step workspaces for a fixed shape.

    upload() builds the index once; step() runs one PQ-HSA decode step and
    dense() the dense split-K baseline, both on the current torch stream.
    """

    def __init__(self, shape: Shape, device="cuda"):
        load()
        self.shape = shape
        self.device = torch.device(device)
        nb = index_bytes(shape)
        if nb == 0:
            raise PQHSAError("pqhsa_index_bytes", 1)
        self.index = torch.empty(nb, dtype=torch.uint8, device=self.device)
        # zero-filled once: the step keeps per-head counters here and leaves
        # them cleared for the next step
        self.workspace = torch.zeros(workspace_bytes(shape, False), dtype=torch.uint8,
                                     device=self.device)
        self._dense_ws = None
        self._events = None
        self.max_selected = max_selected(shape)

    def upload(self, centroids, codebooks, list_ids, codes, n_indexed, v_cache, block_table,
               stream=None):
        ws = torch.empty(max(upload_workspace_bytes(self.shape), 1), dtype=torch.uint8,
                         device=self.device)
        upload_index(self.shape, centroids, codebooks, list_ids, codes, n_indexed, v_cache,
                     block_table, self.index, ws, stream)
        self._upload_ws = ws          # keep alive until the stream has used it

    def append(self, k_cache, v_cache, block_table, new_n_indexed, max_new, list_ids, codes,
               stream=None):
        """Add tokens [n_indexed, new_n_indexed) of each sequence to the index:
        their list ids and codes are written into the token-order `list_ids`
        and `codes` (the arrays the index was uploaded from)."""
        ws = torch.empty(max(append_workspace_bytes(self.shape), 1), dtype=torch.uint8,
                         device=self.device)
        append_tokens(self.shape, self.index, k_cache, v_cache, block_table, new_n_indexed,
                      max_new, list_ids, codes, ws, stream)
        self._append_ws = ws          # keep alive until the stream has used it

    def step(self, q, k_cache, v_cache, block_table, context_lens, out=None, selected=False,
             lse=False, stream=None, staged=False, variant=None):
        """One decode step.  staged=True runs the six staged kernels instead
        of whatever pqhsa_decode_step would choose (for cross-checks);
        variant runs that variant of pqhsa_decode_step_profiled instead."""
        s = self.shape
        if out is None:
            out = torch.empty(s.batch, s.num_q_heads, 128, dtype=torch.float32, device=self.device)
        # -1 marks unused slots; with a zero budget the library writes none
        sel = (torch.full((s.batch, s.num_kv_heads, max(self.max_selected, 1)), -1,
                          dtype=torch.int32, device=self.device) if selected else None)
        ls = torch.empty(s.batch, s.num_q_heads, dtype=torch.float32, device=self.device) if lse else None
        if staged or variant is not None:
            if self._events is None:
                self._events = [HipEvent() for _ in range(2 * NUM_STAGES)]
            decode_step_profiled(s, self.index, q, k_cache, v_cache, block_table, context_lens,
                                 out, self.workspace, self._events,
                                 variant=VARIANT_STAGED if staged else variant,
                                 selected=sel, lse=ls, stream=stream)
        else:
            decode_step(s, self.index, q, k_cache, v_cache, block_table, context_lens, out,
                        self.workspace, selected=sel, lse=ls, stream=stream)
        return out, sel, ls

    def flags(self, clear: bool = False) -> int:
        """The workspace's status word (bit 0: a fused-step barrier wait ran
        out), through pqhsa_step_flags; clear=True also readies the workspace
        for the next step.  Synchronises the current stream."""
        return step_flags(self.shape, self.workspace, clear=clear)

    def dense_workspace(self):
        if self._dense_ws is None:
            self._dense_ws = torch.empty(workspace_bytes(self.shape, True), dtype=torch.uint8,
                                         device=self.device)
        return self._dense_ws

    def dense(self, q, k_cache, v_cache, block_table, context_lens, out=None, lse=False,
              stream=None):
        s = self.shape
        if out is None:
            out = torch.empty(s.batch, s.num_q_heads, 128, dtype=torch.float32, device=self.device)
        ls = torch.empty(s.batch, s.num_q_heads, dtype=torch.float32, device=self.device) if lse else None
        dense_decode_step(s, q, k_cache, v_cache, block_table, context_lens, out,
                          self.dense_workspace(), lse=ls, stream=stream)
        return out, ls


class ReuseDecoder:
    """Dense decode attention with query reuse: owns the per-head query rings
    (kept across steps) and the step's workspace."""

    def __init__(self, shape: Shape, window: int = 1024, max_dist2: float = 1.0,
                 device="cuda"):
        load()
        self.shape, self.window, self.max_dist2, self.device = shape, int(window), max_dist2, device
        nb = reuse_buffer_bytes(shape, window)
        if nb == 0:
            raise PQHSAError("pqhsa_reuse_buffer_bytes", 1)
        self.rings = torch.zeros(nb, dtype=torch.uint8, device=device)
        self.workspace = torch.empty(reuse_workspace_bytes(shape, window), dtype=torch.uint8,
                                     device=device)
        self.layout = reuse_layout(shape, window)

    def clear(self, seq_begin: int = 0, seq_end=None, stream=None):
        reuse_clear(self.shape, self.window, self.rings, seq_begin, seq_end, stream=stream)

    def step(self, q, q_search, k_cache, v_cache, block_table, context_lens, out=None,
             lse=False, report=False, events=None, stream=None):
        """One step; returns (out, lse or None, reused slot or None, min d2 or None)."""
        s = self.shape
        BQ = (s.batch, s.num_q_heads)
        if out is None:
            out = torch.empty(*BQ, 128, dtype=torch.float32, device=self.device)
        ls = torch.empty(*BQ, dtype=torch.float32, device=self.device) if lse else None
        slot = torch.empty(*BQ, dtype=torch.int32, device=self.device) if report else None
        d2 = torch.empty(*BQ, dtype=torch.float32, device=self.device) if report else None
        reuse_decode_step(s, self.window, self.max_dist2, q, q_search, k_cache, v_cache,
                          block_table, context_lens, self.rings, out, self.workspace, lse=ls,
                          reused_slot=slot, min_dist2=d2, events=events, stream=stream)
        return out, ls, slot, d2

    def ring(self, name: str):
        """A view of one ring array: "search" (int16 bf16 bits), "states"
        (float32 [.., 132]), "context" or "count" (int32)."""
        s, W = self.shape, self.window
        BQ = s.batch * s.num_q_heads
        off = getattr(self.layout, name)
        if name == "search":
            return self.rings[off:off + BQ * W * 256].view(torch.int16).view(s.batch, s.num_q_heads, W, 128)
        if name == "states":
            return self.rings[off:off + BQ * W * 528].view(torch.float32).view(s.batch, s.num_q_heads, W, 132)
        if name == "context":
            return self.rings[off:off + BQ * W * 4].view(torch.int32).view(s.batch, s.num_q_heads, W)
        return self.rings[off:off + BQ * 4].view(torch.int32).view(s.batch, s.num_q_heads)
