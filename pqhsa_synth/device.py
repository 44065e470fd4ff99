"""Stage seeded inputs in device memory (paged caches, block table, index arrays).

Copies and layout only; nothing here computes what the attention method
computes.
"""
from __future__ import annotations

import numpy as np
import torch

from .gen import PAGE_SIZE, StepInputs, page_layout, to_paged


def _t(a: np.ndarray, device):
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def stage(inp: StepInputs, device="cuda", page_seed: int = 0, spare_pages: int = 0,
          max_context: int | None = None):
    """Return (tensors, shape_kwargs) for one step's inputs.

    tensors: q, k_cache, v_cache (int16 bf16 bits), block_table, context_lens,
    n_indexed (int32), centroids, codebooks (float32), list_ids (int32) and
    codes (uint8) padded to max_context.  shape_kwargs are the keyword
    arguments of ivf_pq_sparse_amd.make_shape.
    """
    B, Hq, Hkv = inp.batch, inp.num_q_heads, inp.num_kv_heads
    cap = int(inp.context_lens.max()) if max_context is None else int(max_context)
    table, num_pages = page_layout(inp.context_lens, PAGE_SIZE, seed=page_seed,
                                   spare_pages=spare_pages)
    max_pages = max(table.shape[1], (cap + PAGE_SIZE - 1) // PAGE_SIZE)
    if table.shape[1] < max_pages:
        table = np.concatenate([table, np.full((B, max_pages - table.shape[1]), -1, np.int32)], 1)
    kc = to_paged(inp.k_bits, inp.context_lens, table, num_pages)
    vc = to_paged(inp.v_bits, inp.context_lens, table, num_pages)
    Tm = inp.list_ids.shape[2]
    lists = np.zeros((B, Hkv, cap), np.int32)
    codes = np.zeros((B, Hkv, cap, 16), np.uint8)
    n = min(Tm, cap)
    lists[:, :, :n] = inp.list_ids[:, :, :n]
    codes[:, :, :n] = inp.codes[:, :, :n]
    tens = dict(
        q=_t(inp.q_bits, device), k_cache=_t(kc, device), v_cache=_t(vc, device),
        block_table=_t(table, device), context_lens=_t(inp.context_lens.astype(np.int32), device),
        n_indexed=_t(inp.n_indexed.astype(np.int32), device),
        centroids=_t(inp.centroids, device), codebooks=_t(inp.codebooks, device),
        list_ids=_t(lists, device), codes=_t(codes, device))
    shape_kw = dict(batch=B, num_q_heads=Hq, num_kv_heads=Hkv, num_pages=num_pages,
                    max_pages_per_seq=max_pages, max_context=cap, num_lists=inp.num_lists,
                    n_sink=inp.n_sink, n_recent=inp.n_recent, budget_bp=inp.budget_bp,
                    scale=float(inp.scale))
    return tens, shape_kw
