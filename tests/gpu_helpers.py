"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
and compare with the float64 oracle under the stated tolerances.

Tolerances (fixed by the method's accuracy criteria):
  * selected set: identical, except tokens whose oracle key lies within
    1e-5 relative of the k-th largest candidate key (near ties may swap);
  * outputs: compared with the oracle recomputed on the GPU's own selected
    set, within 2e-3 max-abs and 1e-3 mean-relative (sum|diff| / sum|ref|);
  * log-sum-exp: 1e-4 absolute (fp32 accumulation of ~1e5 terms).
"""
from __future__ import annotations

import numpy as np
import torch

import ivf_pq_sparse_amd as pq
from pqhsa_synth.device import stage

SEL_BAND = 1e-5
ATOL_MAX = 2e-3
RTOL_L1 = 1e-3
LSE_ATOL = 1e-4


def log(msg):
    print(msg, flush=True)


def poison_workspace(dec):
    """Fill the decode workspace with 0xFF bytes (NaN as floats, -1 as
    integers) except the regions a step expects cleared (histogram and the
    fused step's counters), so that a read of anything the step did not write
    first shows up in the outputs."""
    lay = pq.workspace_layout(dec.shape)
    ws = dec.workspace
    ws.fill_(0xFF)
    ws[lay.hist:lay.hist + lay.hist_bytes].zero_()
    ws[lay.counters:lay.counters + lay.counters_bytes].zero_()
    torch.cuda.synchronize()


def run_gpu(inp, dense=False, want_selected=True, page_seed=0, spare_pages=0, max_context=None,
            staged=False, background=True, poison=False, variant=None):
    """Stage `inp`, upload the index and run one step; return numpy results.
    staged=True runs the six staged kernels instead of the default path;
    background=False sets exact_only (no background term); poison=True fills
    the workspace's scratch with NaN bytes first; variant runs that variant
    of the profiled entry point."""
    tens, kw = stage(inp, "cuda", page_seed=page_seed, spare_pages=spare_pages,
                     max_context=max_context)
    shape = pq.make_shape(**kw, exact_only=0 if background else 1)
    dec = pq.PQHSADecoder(shape)
    if poison:
        poison_workspace(dec)
    if dense:
        out, lse = dec.dense(tens["q"], tens["k_cache"], tens["v_cache"], tens["block_table"],
                             tens["context_lens"], lse=True)
        torch.cuda.synchronize()
        return dict(O=out.cpu().numpy().astype(np.float64), lse=lse.cpu().numpy(), shape=shape,
                    dec=dec, tens=tens)
    dec.upload(tens["centroids"], tens["codebooks"], tens["list_ids"], tens["codes"],
               tens["n_indexed"], tens["v_cache"], tens["block_table"])
    out, sel, lse = dec.step(tens["q"], tens["k_cache"], tens["v_cache"], tens["block_table"],
                             tens["context_lens"], selected=want_selected, lse=True, staged=staged,
                             variant=variant)
    torch.cuda.synchronize()
    assert dec.flags() == 0, "a barrier wait of the fused step timed out"
    res = dict(O=out.cpu().numpy().astype(np.float64), lse=lse.cpu().numpy(), shape=shape,
               dec=dec, tens=tens)
    if want_selected:
        s = sel.cpu().numpy()
        res["selected"] = {(b, h): s[b, h][s[b, h] >= 0].astype(np.int64)
                           for b in range(shape.batch) for h in range(shape.num_kv_heads)}
    return res


def kth_key(kappa, candidates, k):
    if k <= 0:
        return None
    vals = np.sort(kappa[candidates])[::-1]
    return vals[k - 1]


def check_selection(gpu_sel, ref, heads=None):
    """GPU set vs the oracle's: same size; differences only inside the tie band.
    Returns the number of near-tie differences."""
    import oracle as orc_pkg  # noqa: F401  (test infrastructure)
    diffs = 0
    for key in (ref["selected"] if heads is None else heads):
        g = np.asarray(gpu_sel[key])
        o = np.asarray(ref["selected"][key])
        assert np.all(np.diff(g) > 0), f"{key}: GPU selection not strictly ascending"
        assert g.size == o.size, f"{key}: GPU selected {g.size}, oracle {o.size}"
        sym = np.setxor1d(g, o)
        if sym.size:
            kap, cand, k = ref["kappa"][key], ref["candidates"][key], ref["k"][key]
            thr = kth_key(kap, cand, k)
            band = SEL_BAND * abs(thr)
            far = sym[np.abs(kap[sym] - thr) > band]
            assert far.size == 0, (f"{key}: selection differs outside the tie band at "
                                   f"{far[:8].tolist()} (kth={thr}, keys={kap[far[:8]].tolist()})")
            assert np.all(np.isin(g, cand)), f"{key}: GPU selected a non-candidate"
            diffs += sym.size
    return diffs


def check_output(O_gpu, O_ref, what=""):
    err = np.abs(O_gpu - O_ref)
    l1 = err.sum() / max(np.abs(O_ref).sum(), 1e-300)
    assert np.all(np.isfinite(O_gpu)), f"{what}: non-finite GPU output"
    assert err.max() <= ATOL_MAX, f"{what}: max-abs {err.max():.3e} > {ATOL_MAX}"
    assert l1 <= RTOL_L1, f"{what}: mean-relative {l1:.3e} > {RTOL_L1}"
    return err.max(), l1


def oracle_with_details(inp, heads=None, background=True):
    """Oracle step plus per-head keys/candidates for the selection check."""
    import oracle
    from oracle import pqhsa_oracle as orc
    out = oracle.decode_step(inp, heads=heads, background=background)
    kap, cand = {}, {}
    B, Hkv = inp.batch, inp.num_kv_heads
    G = inp.num_q_heads // Hkv
    todo = [(b, h) for b in range(B) for h in range(Hkv)] if heads is None else list(heads)
    for b, h in todo:
        T, Ti = int(inp.context_lens[b]), int(inp.n_indexed[b])
        q = orc.bf16_to_f64(inp.q_bits[b, h * G:(h + 1) * G])
        qc, lut = orc.lut_tables(q, inp.centroids[b, h].astype(np.float64),
                                 inp.codebooks[b, h].astype(np.float64), inp.scale)
        s = orc.approx_logits(qc, lut, inp.list_ids[b, h, :Ti], inp.codes[b, h, :Ti])
        kap[(b, h)] = s.max(axis=0) if Ti else np.zeros(0)
        cand[(b, h)] = orc.partition(T, Ti, inp.n_sink, inp.n_recent)[1]
    out["kappa"], out["candidates"] = kap, cand
    return out


def parity(inp, heads=None, what="", max_context=None, page_seed=0, staged=False,
           background=True, poison=False):
    """Full check of one step: selection within band, outputs against the
    oracle recomputed with the GPU's set, and the log-sum-exp."""
    log(f"[parity] {what}: B={inp.batch} Hq={inp.num_q_heads} Hkv={inp.num_kv_heads} "
        f"T={inp.context_lens.tolist()} L={inp.num_lists} bp={inp.budget_bp} "
        f"{'staged' if staged else 'default'}{'' if background else ' exact-only'}"
        f"{' poisoned workspace' if poison else ''}")
    g = run_gpu(inp, max_context=max_context, page_seed=page_seed, staged=staged,
                background=background, poison=poison)
    return check_result(g, inp, heads=heads, what=what, background=background)


def check_result(g, inp, heads=None, what="", background=True):
    """Check a GPU step result (as run_gpu returns it) against the oracle on
    `heads` (all (sequence, KV head) pairs if None)."""
    import oracle
    ref = oracle_with_details(inp, heads=heads, background=background)
    nd = check_selection(g["selected"], ref, heads=heads)
    sel = {k: g["selected"][k] for k in ref["selected"]}
    again = oracle.decode_step(inp, selected=sel, heads=heads, background=background)
    G = inp.num_q_heads // inp.num_kv_heads
    todo = sorted(ref["selected"])
    rows = [(b, h * G + gg) for b, h in todo for gg in range(G)]
    bi = np.array([r[0] for r in rows]); qi = np.array([r[1] for r in rows])
    mx, l1 = check_output(g["O"][bi, qi], again["O"][bi, qi], what)
    with np.errstate(divide="ignore"):
        lse_ref = again["m"] + np.log(again["denom"])
    gl, rl = g["lse"][bi, qi], lse_ref[bi, qi]
    # an empty sequence has lse = -inf on both sides
    both_empty = np.isneginf(gl) & np.isneginf(rl)
    lse_err = np.abs(np.where(both_empty, 0.0, gl) - np.where(both_empty, 0.0, rl)).max()
    assert lse_err <= LSE_ATOL, f"{what}: lse error {lse_err:.3e}"
    log(f"[parity] {what}: ok max-abs={mx:.2e} l1={l1:.2e} lse={lse_err:.2e} near-tie diffs={nd}")
    return g, ref, again
