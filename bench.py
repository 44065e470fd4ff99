"""Benchmark: one PQ-HSA decode step of one attention layer on one MI355X.

Default workload: Llama-3.1-8B-like layer (32 query heads, 8 KV heads,
head_dim 128), batch 1, context 131072, IVF 512 lists, PQ 16x8, budget 1 %,
sink 4, recent 128, unindexed tail 256; seeded synthetic data (pqhsa_synth).

A step is the whole path: tables, code scan, top-k, exact split-K with the
background term, merge.  Inputs are resident in HBM before timing starts.
Steps rotate over several copies of the layer (each with its own page
permutation and index buffer) whose total size exceeds the 256 MB Infinity
Cache, so that every step reads from HBM.  The dense split-K decode runs on
the same copies for the speed-up.  Per-stage durations come from HIP events
recorded around each kernel launch on the step's stream.

Prints one JSON line (see the keys below); progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
GATHER_ROWS = 1 << 21          # the gather calibration: rows picked at random
GATHER_ROW_BYTES = 256
METRIC = "µs/decode step/layer @128K, 1% budget; HBM GB/s vs peak; × vs dense split-K"


def cpu_model():
    """The host CPU's model name, or None."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=256)
    p.add_argument("--warmup", type=int, default=32)
    p.add_argument("--workload", type=int, default=2)
    p.add_argument("--layers", type=int, default=0, help="layer copies (0 = enough to exceed MALL)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-dense", action="store_true")
    p.add_argument("--no-graph", action="store_true",
                   help="skip the graph-replayed timing (profiled runs)")
    p.add_argument("--no-other-workloads", action="store_true",
                   help="skip the 8K, 32K, 16 x 128K and 512K lines beside the main workload")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run one plain device copy of known size (for counter scaling)")
    p.add_argument("--sweep", choices=["configs", "budget", "context", "append", "reuse"],
                   help="print a markdown table of a sweep instead of the JSON line")
    p.add_argument("--summarize-profile", nargs=4, metavar=("TRACE", "FETCH", "WRITE", "OUT"),
                   help="write the markdown summary of three rocprofv3 output folders and exit")
    p.add_argument("--summarize-counters", nargs=2, metavar=("PMC_DIR", "OUT"),
                   help="write the markdown table of one rocprofv3 --pmc run and exit")
    p.add_argument("--profile-command", default="",
                   help="the command line recorded in the summary")
    return p.parse_args()


def algorithmic_bytes(inp, n_rows_per_head, k_sel, n_parts):
    """Bytes the method must move per step: in total (the step) and per kernel.

    Step total (the method's own data, scratch not counted): per indexed token
    and KV head 16 B of PQ codes and a 2 B list id; 512 B of bf16 K+V per
    exactly attended row; per KV head the fp32 cluster means and centroids
    (512 B per cluster each) and codebooks (16*256*8*4 B); q and O.

    Per kernel (what one launch must read and write at least, scratch
    included, each array once):
      tables:  q, codebooks, centroids; writes LUT (16*256*G*4 B) and QC (L*G*4 B)
      scan:    per indexed entry 16 B codes + 4 B position read and a 4 B key
               written; per head LUT + QC read, cluster bins (L*G*8 B) written
      collect: per indexed entry the 4 B key; per head the 16 KB histogram;
               writes (position, cluster, G weights) of the k chosen entries
      select:  reads those k records; writes the exact row list (4 B per row),
               the selected positions (4 B each) and selected weights (L*G*8 B)
      attend:  512 B K+V + 4 B row id per exact row; per head the means
               (L*512 B), bins and selected weights; writes the partials
      merge:   reads the partials (132*4 B each), writes O (512 B per q head)
      fused:   the whole step in one kernel, so the step total (its scratch
               stays mostly in L2 and is not counted; its position stream and
               page-table reads are the layout's, not the method's, and are
               reported apart as `fused_layout`: 4 B per indexed entry and per
               exact row instead of the 2 B list id)
    """
    B, Hkv, Hq = inp.batch, inp.num_kv_heads, inp.num_q_heads
    G, L = Hq // Hkv, inp.num_lists
    BH = B * Hkv
    n_idx = int(np.sum(inp.n_indexed)) * Hkv
    rows = int(n_rows_per_head.sum())
    ksum = int(k_sel.sum())
    lut, qc, bins = 16 * 256 * G * 4, L * G * 4, L * G * 8
    partials = B * Hq * n_parts * 132 * 4
    rec = 8 + 4 * G
    total = (n_idx * 18 + rows * 512 + BH * (2 * L * 512 + 16 * 256 * 8 * 4)
             + B * Hq * 128 * (2 + 4))
    k = {
        "fused": total,
        "fused_layout": (n_idx * (16 + 4) + rows * (512 + 4) + BH * (16 * 256 * 8 * 4 + 2 * L * 512)
                         + B * Hq * (256 + 512)),
        "tables": B * Hq * 256 + BH * (16 * 256 * 8 * 4 + L * 512 + lut + qc),
        "scan": n_idx * (16 + 4 + 4) + BH * (lut + qc + bins + (L + 1) * 4),
        "collect": n_idx * 4 + BH * 4096 * 4 + ksum * rec,
        "select": ksum * rec + rows * 4 + ksum * 4 + BH * bins,
        "attend": rows * (512 + 4) + BH * (L * 512 + 2 * bins) + partials,
        "merge": partials + B * Hq * 512,
    }
    return total, k


# ------------------------------------------------------------------ counters
def source_digest():
    """SHA-256 over the kernel sources: counter figures are valid only for the
    sources they were taken on."""
    import hashlib
    h = hashlib.sha256()
    d = os.path.join(ROOT, "ivf_pq_sparse_amd", "csrc")
    for f in sorted(os.listdir(d)):
        if f.endswith((".hip", ".hpp", ".h", ".cpp")):
            h.update(f.encode())
            h.update(open(os.path.join(d, f), "rb").read())
    h.update(open(os.path.join(ROOT, "include", "pqhsa.h"), "rb").read())
    return h.hexdigest()


def _short_kernel(name):
    base = name.split("(")[0].replace("void ", "")
    if base.startswith("pqhsa::"):
        base = base[len("pqhsa::"):]
    return base.replace(" ", "")


def summarize_profile(trace_dir, fetch_dir, write_dir, out, command):
    """Write the markdown summary of one rocprofv3 kernel-trace run and two
    counter runs (FETCH_SIZE, WRITE_SIZE) of the same bench command.  The
    counters are scaled by what they read for the largest plain device copy
    in the run (`--copy-calibration`: 1 GiB read, 1 GiB written)."""
    import csv
    import glob

    def rows(d, pat):
        f = glob.glob(os.path.join(d, pat))
        if not f:
            raise SystemExit(f"no {pat} under {d}")
        return list(csv.DictReader(open(f[0])))

    stats = rows(trace_dir, "*kernel_stats.csv")
    counters = {}
    copy_kib = {}
    gather_kib = {}
    for d, cname in ((fetch_dir, "FETCH_SIZE"), (write_dir, "WRITE_SIZE")):
        per = {}
        for r in rows(d, "*counter_collection.csv"):
            if r["Counter_Name"] != cname:
                continue
            v = float(r["Counter_Value"])
            if r["Kernel_Name"].startswith("__amd_rocclr_copyBuffer"):
                copy_kib[cname] = max(copy_kib.get(cname, 0.0), v)
            if "vectorized_gather_kernel" in r["Kernel_Name"]:
                gather_kib[cname] = max(gather_kib.get(cname, 0.0), v)
            per.setdefault(_short_kernel(r["Kernel_Name"]), []).append(v)
        counters[cname] = {k: (float(np.mean(v)), len(v)) for k, v in per.items()}
    gib_kib = float(1 << 20)
    scale = {c: gib_kib / copy_kib[c] for c in copy_kib}
    lines = ["# rocprofv3 summary: PQ-HSA decode step kernels", "",
             "Command (run from the repository root; three runs of the same bench command):", "",
             "```", command, "```", "",
             f"source_sha256: {source_digest()}", "",
             "Copy calibration (largest `__amd_rocclr_copyBuffer` dispatch, 1 GiB read + 1 GiB "
             "written):", ""]
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        if c in copy_kib:
            lines.append(f"- {c}: {copy_kib[c]:.1f} KiB counted for {gib_kib:.0f} KiB moved: "
                         f"scale x{scale[c]:.4f}")
    if gather_kib:
        g_read = GATHER_ROWS * (GATHER_ROW_BYTES + 8) / 1024.0
        g_write = GATHER_ROWS * GATHER_ROW_BYTES / 1024.0
        lines += ["", f"Gather check (largest `vectorized_gather_kernel` dispatch, torch's index_select: {GATHER_ROWS} random rows of "
                  f"{GATHER_ROW_BYTES} B and their 8 B indices read, the rows written):", ""]
        for c, moved in (("FETCH_SIZE", g_read), ("WRITE_SIZE", g_write)):
            if c in gather_kib:
                lines.append(f"- {c}: {gather_kib[c]:.1f} KiB counted for {moved:.0f} KiB moved: "
                             f"scale x{moved / gather_kib[c]:.4f}")
    lines += ["", "| kernel | calls | avg ns | min ns | max ns | FETCH KiB/dispatch | "
              "WRITE KiB/dispatch | scaled MB/dispatch (read + write) |",
              "|---|---|---|---|---|---|---|---|"]
    for r in stats:
        k = _short_kernel(r["Name"])
        if not (k.startswith("k_") or k.startswith("__amd_rocclr_copyBuffer")):
            continue
        f = counters.get("FETCH_SIZE", {}).get(k)
        w = counters.get("WRITE_SIZE", {}).get(k)
        mb = ""
        if f and w and "FETCH_SIZE" in scale and "WRITE_SIZE" in scale:
            mb = f"{(f[0] * scale['FETCH_SIZE'] + w[0] * scale['WRITE_SIZE']) * 1024 / 1e6:.3f}"
        lines.append(f"| {k} | {r['Calls']} | {float(r['AverageNs']):.0f} | {r['MinNs']} | "
                     f"{r['MaxNs']} | {f[0] if f else float('nan'):.1f} | "
                     f"{w[0] if w else float('nan'):.1f} | {mb} |")
    lines += ["", "Machine-readable (kernel, avg_ns, scaled_bytes_per_dispatch):", "", "```"]
    for r in stats:
        k = _short_kernel(r["Name"])
        f = counters.get("FETCH_SIZE", {}).get(k)
        w = counters.get("WRITE_SIZE", {}).get(k)
        if k.startswith("k_") and f and w and "FETCH_SIZE" in scale and "WRITE_SIZE" in scale:
            b = (f[0] * scale["FETCH_SIZE"] + w[0] * scale["WRITE_SIZE"]) * 1024
            lines.append(f"{k} {float(r['AverageNs']):.0f} {b:.0f}")
    lines += ["```", ""]
    open(out, "w").write("\n".join(lines))
    print(f"wrote {out}", file=sys.stderr)


def summarize_counters(counter_dir, out, command, kernels):
    """Markdown table of the mean value per dispatch of every counter of one
    rocprofv3 --pmc run, for the named kernels (prefix match)."""
    import csv
    import glob
    f = glob.glob(os.path.join(counter_dir, "*counter_collection.csv"))
    if not f:
        raise SystemExit(f"no counter_collection.csv under {counter_dir}")
    acc = {}
    for r in csv.DictReader(open(f[0])):
        k = _short_kernel(r["Kernel_Name"])
        if not any(k.startswith(x) for x in kernels):
            continue
        acc.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    names = sorted({c for v in acc.values() for c in v})
    lines = ["# rocprofv3 counters per dispatch (mean over dispatches)", "",
             "Command (run from the repository root):", "", "```", command, "```", "",
             f"source_sha256: {source_digest()}", "",
             "| kernel | dispatches | " + " | ".join(names) + " |",
             "|---|---|" + "---|" * len(names)]
    for k in sorted(acc):
        n = max(len(v) for v in acc[k].values())
        lines.append(f"| {k} | {n} | " + " | ".join(
            f"{np.mean(acc[k][c]):.4g}" if c in acc[k] else "" for c in names) + " |")
    open(out, "w").write("\n".join(lines) + "\n")
    print(f"wrote {out}", file=sys.stderr)


def stored_traffic(path):
    """{kernel: (avg_ns, bytes per dispatch)} from a committed summary, or None
    when it is missing or was taken on other kernel sources."""
    if not os.path.exists(path):
        return None
    text = open(path).read()
    if f"source_sha256: {source_digest()}" not in text:
        return None
    out = {}
    block = text.split("Machine-readable", 1)[-1].split("```")[1]
    for ln in block.strip().splitlines():
        k, ns, b = ln.split()
        out[k] = (float(ns), float(b))
    return out


def kernel_of_stage(stage, G, n_parts=0):
    """Kernel symbol (as rocprofv3 shortens it) that a stage launches (the
    merge kernel's template argument is its number of part groups)."""
    ng = 2 if n_parts <= 64 else 4 if n_parts <= 128 else 8
    return {"fused": f"k_fused<{G}>",
            "tables": f"k_tables<{G}>", "scan": f"k_scan<{G}>", "collect": f"k_collect<{G}>",
            "select": f"k_select<{G}>", "attend": f"k_attend<{G},0>",
            "merge": f"k_merge<{ng}>"}[stage]


class Rig:
    """Layer copies of one step's inputs on the GPU (each with its own page
    permutation and index, together larger than the 256 MB Infinity Cache)
    and timed loops over them."""

    def __init__(self, inp, n_layers=0, exact_only=0, max_bytes=60e9, with_index=True):
        import torch

        import ivf_pq_sparse_amd as pq
        from pqhsa_synth.device import stage
        self.torch, self.pq = torch, pq
        tens, kw = stage(inp, "cuda")
        self.shape = pq.make_shape(**kw, exact_only=exact_only)
        kv_bytes = 2 * tens["k_cache"].numel() * 2
        self.kv_bytes = kv_bytes
        n = n_layers or max(2, int(np.ceil(2.5 * 256e6 / (kv_bytes / 17.6 + 1))))
        ix_bytes = pq.index_bytes(self.shape) if with_index else 0
        n = min(n, max(2, int(max_bytes // (kv_bytes + ix_bytes))))
        self.n_layers = n
        self.layers = []
        g = torch.Generator(device="cpu").manual_seed(1234)
        P = self.shape.num_pages
        for _ in range(n):
            perm = torch.randperm(P, generator=g).to("cuda")
            kc = torch.empty_like(tens["k_cache"])
            vc = torch.empty_like(tens["v_cache"])
            kc[perm] = tens["k_cache"]
            vc[perm] = tens["v_cache"]
            bt = tens["block_table"].clone()
            valid = bt >= 0
            bt[valid] = perm[bt[valid].long()].to(torch.int32)
            dec = None
            if with_index:
                dec = pq.PQHSADecoder(self.shape)
                dec.upload(tens["centroids"], tens["codebooks"], tens["list_ids"], tens["codes"],
                           tens["n_indexed"], vc, bt)
            self.layers.append(dict(kc=kc, vc=vc, bt=bt, dec=dec))
        torch.cuda.synchronize()
        del tens["k_cache"], tens["v_cache"]
        self.q, self.ctx = tens["q"], tens["context_lens"]
        if with_index:
            self.ws = self.layers[0]["dec"].workspace
            self.dense_ws = self.layers[0]["dec"].dense_workspace()
        else:
            self.ws = None
            self.dense_ws = torch.empty(pq.workspace_bytes(self.shape, True), dtype=torch.uint8,
                                        device="cuda")
        self.out = torch.empty(self.shape.batch, self.shape.num_q_heads, 128,
                               dtype=torch.float32, device="cuda")

    def step(self, i, dense=False, out=None):
        pq, L_ = self.pq, self.layers[i % self.n_layers]
        out = self.out if out is None else out
        if dense:
            pq.dense_decode_step(self.shape, self.q, L_["kc"], L_["vc"], L_["bt"], self.ctx, out,
                                 self.dense_ws)
        else:
            pq.decode_step(self.shape, L_["dec"].index, self.q, L_["kc"], L_["vc"], L_["bt"],
                           self.ctx, out, self.ws)

    def timed(self, dense, steps, warmup):
        """Average µs per step over `steps` steps after `warmup` untimed ones."""
        torch, pq = self.torch, self.pq
        for i in range(warmup):
            self.step(i, dense)
        torch.cuda.synchronize()
        e0, e1 = pq.HipEvent(), pq.HipEvent()
        stream = torch.cuda.current_stream()
        e0.record(stream)
        for i in range(steps):
            self.step(i, dense)
        e1.record(stream)
        e1.synchronize()
        torch.cuda.synchronize()
        return e0.elapsed_ms(e1) / steps * 1e3


def other_workloads(main_wid, steps=128, warmup=64):
    """The 8K, 32K, 16 x 128K and 512K workloads beside the main one: PQ-HSA and
    dense split-K µs per step on rotated layer copies, the speed-up and the
    step's algorithmic bytes and rate."""
    import torch

    import ivf_pq_sparse_amd as pq
    from pqhsa_synth import WORKLOADS, make_step_inputs
    out = {}
    for wid in (0, 1, 3, 4):
        if wid == main_wid:
            continue
        w = WORKLOADS[wid]
        t0 = time.time()
        inp = make_step_inputs(wid)
        rig = Rig(inp)
        us = rig.timed(False, steps, warmup)
        dus = rig.timed(True, steps, warmup)
        flags = pq.step_flags(rig.shape, rig.ws)
        if flags:
            raise SystemExit(f"workload {wid}: a barrier wait of the fused step ran out")
        k = -(-w["context"] * w["budget_bp"] // 10000)
        n_rows = np.full(w["batch"] * w["num_kv_heads"],
                         w["n_sink"] + k + max(w["n_recent"], w["n_tail"]))
        tot, _ = algorithmic_bytes(inp, n_rows, np.full(n_rows.size, k), 1)
        out[w["name"]] = {"pqhsa_us": us, "dense_us": dus, "speedup_vs_dense": dus / us,
                          "step_alg_bytes": tot, "step_alg_gbps": tot / (us * 1e-6) / 1e9,
                          "dense_gbps": rig.kv_bytes / (dus * 1e-6) / 1e9,
                          "layer_copies": rig.n_layers, "steps": steps}
        log(f"workload {wid} ({w['name']}): PQ-HSA {us:.1f} µs, dense {dus:.1f} µs "
            f"({time.time() - t0:.0f} s)")
        del rig, inp
        torch.cuda.empty_cache()
    return out


def reuse_sweep(steps, warmup, window=1024):
    """Query reuse at the 128K Llama-3.1-8B layer shape: every layer copy keeps
    its own rings; step i runs all copies at context T0 + i with search
    vectors that repeat with period `dist` (exact repeats, so every head
    reuses the entry of `dist` steps earlier: a suffix of `dist` tokens).
    "none" sets a negative threshold (search, then full attention); dense is
    the plain split-K step on the same copies."""
    import torch

    import ivf_pq_sparse_amd as pq
    from pqhsa_synth import f32_to_bf16_bits, make_step_inputs
    n_total = 1100 + warmup + steps + 16
    T_end = 131072
    inp = make_step_inputs(2, context_lens=[T_end], num_lists=8, n_tail=0)
    rig = Rig(inp, with_index=False)
    shape, B, Hq = rig.shape, rig.shape.batch, rig.shape.num_q_heads
    rng = np.random.default_rng(5)
    topics = rng.standard_normal((1024, B, Hq, 128)).astype(np.float32)
    qbits = torch.from_numpy(f32_to_bf16_bits(topics).view(np.int16)).cuda()
    decs = [pq.ReuseDecoder(shape, window=window, max_dist2=0.5) for _ in range(rig.n_layers)]
    out = torch.empty(B, Hq, 128, dtype=torch.float32, device="cuda")
    ctxs = [torch.tensor([T_end - n_total + i] * B, dtype=torch.int32, device="cuda")
            for i in range(n_total)]
    slot = torch.empty(B, Hq, dtype=torch.int32, device="cuda")
    d2 = torch.empty(B, Hq, dtype=torch.float32, device="cuda")
    evs = [pq.HipEvent() for _ in range(6)]
    stream = torch.cuda.current_stream()
    dense_us = rig.timed(True, steps * rig.n_layers // 4, warmup)
    print(f"K/V copies: {rig.n_layers}; window {window}; dense split-K step {dense_us:.1f} µs")
    print()
    print("| reuse distance (tokens) | heads reusing | wall µs per layer-step | kernel µs | "
          "dense µs | speed-up (kernels) | search µs | attend µs | merge µs |")
    print("|---|---|---|---|---|---|---|---|---|")
    for dist in (1, 8, 64, 256, 1000, "none"):
        period = 1000 if dist == "none" else dist
        for d in decs:
            d.clear()
            d.max_dist2 = -1.0 if dist == "none" else 0.5

        def run(i, layer, events=None):
            d = decs[layer]
            L_ = rig.layers[layer]
            q = qbits[i % period]
            d.step(q, q, L_["kc"], L_["vc"], L_["bt"], ctxs[i], out=out, events=events)

        n_warm = period + warmup
        for i in range(n_warm):
            for layer in range(rig.n_layers):
                run(i, layer)
        torch.cuda.synchronize()
        e0, e1 = pq.HipEvent(), pq.HipEvent()
        e0.record(stream)
        for i in range(n_warm, n_warm + steps):
            for layer in range(rig.n_layers):
                run(i, layer)
        e1.record(stream)
        e1.synchronize()
        us = e0.elapsed_ms(e1) * 1e3 / (steps * rig.n_layers)
        # kernel split on further steps, and the share of heads reusing
        ks = np.zeros(3)
        n_prof = 8
        for j in range(n_prof + 1):     # j = 0: untimed first use of the events
            i = n_warm + steps + j
            layer = j % rig.n_layers
            L_ = rig.layers[layer]
            q = qbits[i % period]
            pq.reuse_decode_step(shape, window, decs[layer].max_dist2, q, q, L_["kc"], L_["vc"],
                                 L_["bt"], ctxs[i], decs[layer].rings, out, decs[layer].workspace,
                                 reused_slot=slot, min_dist2=d2, events=evs)
            for r in range(layer + 1, rig.n_layers):
                run(i, r)
            evs[5].synchronize()
            if j:
                ks += [evs[2 * k].elapsed_ms(evs[2 * k + 1]) * 1e3 for k in range(3)]
        ks /= n_prof
        frac = float((slot >= 0).float().mean())
        kus = float(ks.sum())
        print(f"| {dist} | {frac * 100:.0f} % | {us:.1f} | {kus:.1f} | {dense_us:.1f} | "
              f"{dense_us / kus:.2f} | {ks[0]:.1f} | {ks[1]:.1f} | {ks[2]:.1f} |", flush=True)
        log(f"reuse distance {dist}: {us:.1f} µs per layer-step (dense {dense_us:.1f})")


def sweep(name, steps, warmup):
    """Markdown tables on stdout (progress on stderr):
      configs: every workload, PQ-HSA step and dense split-K step;
      budget:  the 128K workload at budgets 0.25 % .. 100 %, with and without
               the background term, time and output error against dense
               attention on the same inputs;
      context: the 128K workload's layer shape at 8K .. 512K tokens, PQ-HSA
               vs dense split-K (where the index starts to pay);
      append:  index build (whole upload) and update (appending a batch of
               new tokens) at the 128K workload's shape."""
    import torch

    import ivf_pq_sparse_amd as pq
    from pqhsa_synth import WORKLOADS, make_step_inputs
    pq.load()
    rows = []
    if name == "configs":
        print("| workload | B x T | Hq/Hkv | L | k | PQ-HSA µs | dense µs | speed-up | "
              "alg. MB | alg. GB/s |")
        print("|---|---|---|---|---|---|---|---|---|---|")
        for wid in range(5):
            w = WORKLOADS[wid]
            inp = make_step_inputs(wid)
            rig = Rig(inp)
            us = rig.timed(False, steps, warmup)
            dus = rig.timed(True, steps, warmup)
            k = -(-w["context"] * w["budget_bp"] // 10000)
            n_rows = np.full(w["batch"] * w["num_kv_heads"],
                             w["n_sink"] + k + max(w["n_recent"], w["n_tail"]))
            tot, _ = algorithmic_bytes(inp, n_rows, np.full(n_rows.size, k), 1)
            print(f"| {wid} {w['name']} | {w['batch']} x {w['context']} | "
                  f"{w['num_q_heads']}/{w['num_kv_heads']} | {w['num_lists']} | {k} | "
                  f"{us:.1f} | {dus:.1f} | {dus / us:.2f} | {tot / 1e6:.1f} | "
                  f"{tot / (us * 1e-6) / 1e9:.0f} |", flush=True)
            log(f"workload {wid}: {us:.1f} µs, dense {dus:.1f} µs ({rig.n_layers} copies)")
            del rig
            torch.cuda.empty_cache()
    elif name == "budget":
        inp = make_step_inputs(2)
        print("| budget | background | PQ-HSA µs | dense µs | speed-up | max-abs err vs dense | "
              "mean-rel err vs dense |")
        print("|---|---|---|---|---|---|---|")
        for bp in (25, 50, 100, 200, 500, 1000, 10000):
            inp.budget_bp = bp
            for eo in (0, 1):
                rig = Rig(inp, n_layers=0, exact_only=eo)
                us = rig.timed(False, steps, warmup)
                dus = rig.timed(True, steps, warmup)
                o_s = torch.empty_like(rig.out)
                o_d = torch.empty_like(rig.out)
                rig.step(0, False, o_s)
                rig.step(0, True, o_d)
                torch.cuda.synchronize()
                err = (o_s - o_d).abs()
                rel = float(err.sum() / o_d.abs().sum())
                print(f"| {bp / 100:g} % | {'off' if eo else 'on'} | {us:.1f} | {dus:.1f} | "
                      f"{dus / us:.2f} | {float(err.max()):.2e} | {rel:.2e} |", flush=True)
                log(f"budget {bp} bp exact_only={eo}: {us:.1f} µs")
                del rig
                torch.cuda.empty_cache()
    elif name == "context":
        print("| context | L | k | PQ-HSA µs | dense µs | speed-up |")
        print("|---|---|---|---|---|---|")
        for T in (8192, 16384, 32768, 65536, 131072, 262144, 524288):
            L = max(64, T // 256)
            inp = make_step_inputs(2, context_lens=[T], num_lists=L)
            rig = Rig(inp)
            us = rig.timed(False, steps, warmup)
            dus = rig.timed(True, steps, warmup)
            k = -(-T * inp.budget_bp // 10000)
            print(f"| {T} | {L} | {k} | {us:.1f} | {dus:.1f} | {dus / us:.2f} |", flush=True)
            log(f"context {T}: {us:.1f} µs, dense {dus:.1f} µs")
            del rig
            torch.cuda.empty_cache()
    elif name == "append":
        # index build (upload of the whole index) and update (append of a
        # batch of new tokens) at the 128K workload's shape
        from pqhsa_synth.device import stage
        print("| operation | tokens per (seq, KV head) | µs | µs per token per KV head |")
        print("|---|---|---|---|")
        for nb in (0, 16, 64, 256, 1024, 4096):
            inp = make_step_inputs(2, n_tail=max(nb, 256))
            tens, kw = stage(inp, "cuda")
            shape = pq.make_shape(**kw)
            dec = pq.PQHSADecoder(shape)
            Hkv = shape.num_kv_heads
            T = int(inp.context_lens[0])
            e0, e1 = pq.HipEvent(), pq.HipEvent()
            stream = torch.cuda.current_stream()
            times = []
            for rep in range(6):
                lists = tens["list_ids"].clone()
                codes = tens["codes"].clone()
                if nb == 0:
                    n_full = torch.tensor(inp.context_lens, dtype=torch.int32, device="cuda")
                    torch.cuda.synchronize()
                    e0.record(stream)
                    dec.upload(tens["centroids"], tens["codebooks"], lists, codes, n_full,
                               tens["v_cache"], tens["block_table"])
                    e1.record(stream)
                else:
                    n_old = torch.tensor([T - nb], dtype=torch.int32, device="cuda")
                    n_new = torch.tensor([T], dtype=torch.int32, device="cuda")
                    dec.upload(tens["centroids"], tens["codebooks"], lists, codes, n_old,
                               tens["v_cache"], tens["block_table"])
                    torch.cuda.synchronize()
                    e0.record(stream)
                    dec.append(tens["k_cache"], tens["v_cache"], tens["block_table"], n_new,
                               nb, lists, codes)
                    e1.record(stream)
                e1.synchronize()
                if rep:
                    times.append(e0.elapsed_ms(e1) * 1e3)
            us = float(np.median(times))
            what = "upload (build, all tokens)" if nb == 0 else "append"
            ntok = T if nb == 0 else nb
            print(f"| {what} | {ntok} | {us:.1f} | {us / ntok / Hkv:.4f} |", flush=True)
            log(f"{what} {ntok}: {us:.1f} µs")
            del dec, tens
            torch.cuda.empty_cache()
    elif name == "reuse":
        reuse_sweep(steps, warmup)
    else:
        raise SystemExit(f"unknown sweep {name}")


def main():
    args = parse()
    if args.summarize_profile:
        summarize_profile(*args.summarize_profile, command=args.profile_command)
        return
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters, command=args.profile_command,
                           kernels=("k_fused", "k_dense_mfma", "k_attend", "k_scan", "k_merge"))
        return
    if args.sweep:
        sweep(args.sweep, args.steps, args.warmup)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the PQ-HSA step "
              "shards by sequence or KV head with no exchange, so there is no multi-GPU mode",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import ivf_pq_sparse_amd as pq
    from pqhsa_synth import WORKLOADS, make_step_inputs
    from pqhsa_synth.device import stage

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    pq.load()
    w = WORKLOADS[args.workload]
    t0 = time.time()
    inp = make_step_inputs(args.workload)
    log(f"generated workload {args.workload} ({w['name']}) in {time.time() - t0:.1f}s")
    tens, kw = stage(inp, "cuda")
    shape = pq.make_shape(**kw)
    kv_bytes = 2 * tens["k_cache"].numel() * 2
    n_layers = args.layers or max(2, int(np.ceil(2.5 * 256e6 / (kv_bytes / 17.6 + 1))))
    n_layers = min(n_layers, max(2, int(60e9 // (kv_bytes + pq.index_bytes(shape)))))
    log(f"KV cache {kv_bytes / 1e9:.2f} GB per layer; {n_layers} layer copies")

    # layer copies: same logical data, different physical pages and buffers
    layers = []
    g = torch.Generator(device="cpu").manual_seed(1234)
    P = shape.num_pages
    for li in range(n_layers):
        perm = torch.randperm(P, generator=g).to("cuda")
        kc = torch.empty_like(tens["k_cache"])
        vc = torch.empty_like(tens["v_cache"])
        kc[perm] = tens["k_cache"]
        vc[perm] = tens["v_cache"]
        bt = tens["block_table"].clone()
        valid = bt >= 0
        bt[valid] = perm[bt[valid].long()].to(torch.int32)
        dec = pq.PQHSADecoder(shape)
        dec.upload(tens["centroids"], tens["codebooks"], tens["list_ids"], tens["codes"],
                   tens["n_indexed"], vc, bt)
        layers.append(dict(kc=kc, vc=vc, bt=bt, dec=dec))
    torch.cuda.synchronize()
    del tens["k_cache"], tens["v_cache"]
    log("layers staged and indexed")

    ws = layers[0]["dec"].workspace
    dense_ws = layers[0]["dec"].dense_workspace()
    out = torch.empty(shape.batch, shape.num_q_heads, 128, dtype=torch.float32, device="cuda")
    q, ctx = tens["q"], tens["context_lens"]
    stream = torch.cuda.current_stream()

    def step(i, dense=False):
        L_ = layers[i % n_layers]
        if dense:
            pq.dense_decode_step(shape, q, L_["kc"], L_["vc"], L_["bt"], ctx, out, dense_ws)
        else:
            pq.decode_step(shape, L_["dec"].index, q, L_["kc"], L_["vc"], L_["bt"], ctx, out, ws)

    def timed(dense):
        """Mean ms per step over the timed steps (events at both ends only)."""
        for i in range(args.warmup):
            step(i, dense)
        torch.cuda.synchronize()
        e0, e1 = pq.HipEvent(), pq.HipEvent()
        e0.record(stream)
        for i in range(args.steps):
            step(i, dense)
        e1.record(stream)
        e1.synchronize()
        torch.cuda.synchronize()
        return e0.elapsed_ms(e1) / args.steps

    def per_step(dense):
        """µs of each step of a separate pass (at least 64 steps, at most 256)
        with an event recorded after every step on the step stream: the spread
        of single steps, whatever --steps is.  The extra events make each step
        a little slower than in the timed loop."""
        n = min(256, max(64, args.steps))
        marks = [pq.HipEvent() for _ in range(n + 1)]
        torch.cuda.synchronize()
        marks[0].record(stream)
        for i in range(n):
            step(i, dense)
            marks[i + 1].record(stream)
        marks[-1].synchronize()
        return [marks[i].elapsed_ms(marks[i + 1]) * 1e3 for i in range(n)]

    def graph_us(dense):
        """µs per step when `steps` steps are captured once in a HIP graph
        (torch.cuda.graph) and the graph is replayed: the host launch work
        the eager loop pays per step is paid once per replay.  The steps
        clear their own counters in their kernels, so a replay is exact."""
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            for i in range(args.warmup):
                step(i, dense)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(args.steps):
                step(i, dense)
        graph.replay()
        torch.cuda.synchronize()
        e0, e1 = pq.HipEvent(), pq.HipEvent()
        e0.record(stream)
        graph.replay()
        e1.record(stream)
        e1.synchronize()
        torch.cuda.synchronize()
        del graph
        return e0.elapsed_ms(e1) / args.steps * 1e3

    def spread(per):
        if not per:
            return None
        p = np.percentile(per, [10, 50, 90])
        return {"p10_us": float(p[0]), "p50_us": float(p[1]), "p90_us": float(p[2]),
                "steps": len(per), "source": "one event after every step, separate pass"}

    ms = timed(False)
    log(f"PQ-HSA step: {ms * 1e3:.2f} µs")
    step_reps = per_step(False)
    dense_ms = None if args.no_dense else timed(True)
    dense_reps = [] if args.no_dense else per_step(True)
    if dense_ms is not None:
        log(f"dense split-K step: {dense_ms * 1e3:.2f} µs")
    graph_step = None if args.no_graph else graph_us(False)
    graph_dense = None if args.no_graph or args.no_dense else graph_us(True)
    if graph_step is not None:
        log(f"graph-replayed steps: PQ-HSA {graph_step:.2f} µs"
            + (f", dense {graph_dense:.2f} µs" if graph_dense is not None else ""))

    # per-kernel durations: the same steps through the profiled entry point,
    # every kernel with its own start/stop events on the step's stream
    def kernel_us(variant):
        wsv = dense_ws if variant == pq.VARIANT_DENSE else ws
        evs = [[pq.HipEvent() for _ in range(2 * pq.NUM_STAGES)] for _ in range(args.steps)]
        for i in range(args.warmup):
            step(i, variant == pq.VARIANT_DENSE)
        torch.cuda.synchronize()
        nk = 0
        for i in range(args.steps):
            L_ = layers[i % n_layers]
            nk = pq.decode_step_profiled(shape, L_["dec"].index, q, L_["kc"], L_["vc"], L_["bt"],
                                         ctx, out, wsv, evs[i], variant=variant)
        torch.cuda.synchronize()
        t = np.array([[evs[i][2 * k].elapsed_ms(evs[i][2 * k + 1]) * 1e3 for k in range(nk)]
                      for i in range(args.steps)])
        return t.mean(axis=0)

    step_k = kernel_us(pq.VARIANT_DEFAULT)
    fused = len(step_k) == 1
    names = ["fused"] if fused else list(pq.STAGE_NAMES)
    stage_us = step_k
    staged_us = kernel_us(pq.VARIANT_STAGED)
    dense_stage = None if args.no_dense else kernel_us(pq.VARIANT_DENSE)
    log("step kernels µs: " + ", ".join(f"{n}={v:.2f}" for n, v in zip(names, stage_us)))
    log("staged kernels µs: " + ", ".join(f"{n}={v:.2f}" for n, v in zip(pq.STAGE_NAMES,
                                                                          staged_us)))
    if fused and pq.PQHSADecoder.flags(layers[0]["dec"]) != 0:
        raise SystemExit("a barrier wait of the fused step timed out")

    # exact rows and k per head from the last step's workspace
    lay = pq.workspace_layout(shape)
    BH = shape.batch * shape.num_kv_heads
    n_rows = ws[lay.n_rows:lay.n_rows + BH * 4].view(torch.int32).cpu().numpy()
    k_sel = np.array([min(-(-int(inp.context_lens[b]) * inp.budget_bp // 10000),
                          10 ** 9) for b in range(inp.batch) for _ in range(inp.num_kv_heads)])
    step_bytes, kbytes = algorithmic_bytes(inp, n_rows, k_sel, lay.n_parts)

    if args.copy_calibration:
        n = 1 << 28                                   # 1 GiB of fp32
        src = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: {n * 4} bytes read and written")
        # and a gather of known bytes: 2M random rows of 256 B (the step's K/V
        # rows are 256 B runs) and their 8-byte indices read, the rows written
        rows = src.view(-1, GATHER_ROW_BYTES // 4)
        g = torch.Generator(device="cuda").manual_seed(7)
        idx = torch.randperm(rows.shape[0], device="cuda", generator=g)[:GATHER_ROWS]
        torch.cuda.synchronize()
        picked = rows.index_select(0, idx)
        torch.cuda.synchronize()
        log(f"gather calibration: {picked.numel() * 4} bytes of rows gathered")
        del picked, idx

    # dominant kernel (longest average duration) and its roofline over its
    # algorithmic bytes (for the fused kernel, the whole step's: codes, list
    # ids, exact rows, index tables, q and O); traffic from the committed
    # counter summary when it was taken on these kernel sources
    dom = int(np.argmax(stage_us))
    dom_bytes = kbytes[names[dom]]
    achieved = dom_bytes / (stage_us[dom] * 1e-6) / 1e9
    prof = stored_traffic(os.path.join(ROOT, "profiles", f"counters_{w['name']}.md"))
    G = shape.num_q_heads // shape.num_kv_heads
    kname = kernel_of_stage(names[dom], G, lay.n_parts)
    traffic = prof[kname][1] if prof and kname in prof else None
    roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                "traffic_gbps": (traffic / (stage_us[dom] * 1e-6) / 1e9) if traffic else None,
                "kernel": kname, "alg_bytes_per_launch": dom_bytes,
                "launch_us": float(stage_us[dom]),
                "traffic_over_alg": (traffic / dom_bytes) if traffic else None}
    if fused:
        # the layout's own bytes (4 B positions, page-table entries) beside
        roofline["layout_bytes_per_launch"] = kbytes["fused_layout"]
        roofline["frac_over_layout_bytes"] = (kbytes["fused_layout"] / (stage_us[dom] * 1e-6)
                                              / 1e9 / HBM_PEAK_GBS)

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        import resource
        reps = 0
        r0 = resource.getrusage(resource.RUSAGE_SELF)
        t0 = time.time()
        while reps < 1 or (time.time() - t0 < 10.0 and reps < 8):
            oracle.decode_step(inp)
            reps += 1
        wall = time.time() - t0
        r1 = resource.getrusage(resource.RUSAGE_SELF)
        cpu_s = (r1.ru_utime - r0.ru_utime) + (r1.ru_stime - r0.ru_stime)
        cpu = {"value": wall / reps * 1e6, "unit": "µs/step/layer",
               "cores": max(1, int(round(cpu_s / wall))), "kind": "oracle",
               "sample": f"the full step of this workload ({inp.batch * inp.num_kv_heads} KV heads), "
                         f"{reps} repetitions, numpy float64, input generation and index build excluded",
               "host_threads_available": os.cpu_count(), "cpu_model": cpu_model()}
        log(f"oracle: {cpu['value'] / 1e3:.1f} ms/step on ~{cpu['cores']} cores")
        # the same with the numerical libraries held to one thread
        try:
            from threadpoolctl import threadpool_limits
            with threadpool_limits(1):
                t1, reps1 = time.time(), 0
                while reps1 < 1 or (time.time() - t1 < 5.0 and reps1 < 4):
                    oracle.decode_step(inp)
                    reps1 += 1
                cpu["single_thread_value"] = (time.time() - t1) / reps1 * 1e6
            log(f"oracle, one thread: {cpu['single_thread_value'] / 1e3:.1f} ms/step")
        except ImportError:
            cpu["single_thread_value"] = None

    others = None
    if not args.no_other_workloads:
        del layers, ws, dense_ws
        torch.cuda.empty_cache()
        others = other_workloads(args.workload)

    us = ms * 1e3
    rec = {
        "metric": METRIC, "value": us, "unit": "µs/step/layer", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w["name"], "batch": w["batch"], "context": w["context"],
                   "num_q_heads": w["num_q_heads"], "num_kv_heads": w["num_kv_heads"],
                   "head_dim": 128, "num_lists": w["num_lists"], "pq": "16x8 bits",
                   "budget": f"{w['budget_bp'] / 100:g}%", "sink": w["n_sink"],
                   "recent": w["n_recent"], "tail": w["n_tail"], "kv_dtype": "bf16",
                   "page_size": 16, "layer_copies": n_layers},
        "step_us_spread": spread(step_reps),
        "dense_us": dense_ms * 1e3 if dense_ms else None,
        "dense_us_spread": spread(dense_reps),
        "graph_replay_us": ({"step": graph_step, "dense": graph_dense,
                             "source": f"{args.steps} steps captured in one HIP graph, "
                                       "one timed replay"} if graph_step is not None else None),
        "speedup_vs_dense": (dense_ms / ms) if dense_ms else None,
        "step_alg_bytes": step_bytes,
        "step_alg_gbps": step_bytes / (ms * 1e-3) / 1e9,
        "kernel_alg_bytes": kbytes,
        "dense_alg_gbps": (kv_bytes / (dense_ms * 1e-3) / 1e9) if dense_ms else None,
        "kernels_us": {n: float(v) for n, v in zip(names, stage_us)},
        "staged_kernels_us": {n: float(v) for n, v in zip(pq.STAGE_NAMES, staged_us)},
        "dense_kernels_us": ({"splitk": float(dense_stage[0]), "merge": float(dense_stage[1])}
                             if dense_stage is not None else None),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "other_workloads": others,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
