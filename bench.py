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
METRIC = "µs/decode step/layer @128K, 1% budget; HBM GB/s vs peak; × vs dense split-K"


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
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run one plain device copy of known size (for counter scaling)")
    return p.parse_args()


def algorithmic_bytes(inp, n_rows_per_head, k_sel):
    """Bytes the method must move per step (per stage and in total).

    scan:   per indexed entry 16 B codes + 4 B position read, 4 B key written;
            per (b, h) the lookup table and cluster tables.
    exact:  512 B (bf16 K + V row) per exact row, 4 B row index.
    background: cluster means (512 B per cluster), bins, selected codes.
    """
    B, Hkv, Hq = inp.batch, inp.num_kv_heads, inp.num_q_heads
    G, L = Hq // Hkv, inp.num_lists
    n_idx = int(np.sum(inp.n_indexed)) * Hkv
    per_head_tables = 16 * 256 * G * 4 + L * G * 4 + L * G * 8
    scan = n_idx * (16 + 4 + 4) + B * Hkv * per_head_tables
    exact = int(n_rows_per_head.sum()) * (512 + 4)
    background = B * Hkv * (L * 512 + L * G * 8 + L * G * 4) + int(k_sel.sum()) * 16
    tables = B * Hkv * (16 * 256 * 8 * 4 + L * 128 * 4 + per_head_tables) + B * Hq * 256
    io = B * Hq * 128 * 4
    total = scan + exact + background + tables + io
    return dict(scan=scan, exact=exact, background=background, tables=tables, total=total)


def main():
    args = parse()
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

    ms = timed(False)
    log(f"PQ-HSA step: {ms * 1e3:.2f} µs")
    dense_ms = None if args.no_dense else timed(True)
    if dense_ms is not None:
        log(f"dense split-K step: {dense_ms * 1e3:.2f} µs")

    # per-stage durations (events between launches on the same stream)
    nst = pq.NUM_STAGES
    evs = [[pq.HipEvent() for _ in range(nst + 1)] for _ in range(args.steps)]
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    for i in range(args.steps):
        L_ = layers[i % n_layers]
        pq.decode_step_profiled(shape, L_["dec"].index, q, L_["kc"], L_["vc"], L_["bt"], ctx, out,
                                ws, evs[i])
    torch.cuda.synchronize()
    stage_us = np.zeros(nst)
    for i in range(args.steps):
        for s in range(nst):
            stage_us[s] += evs[i][s].elapsed_ms(evs[i][s + 1]) * 1e3
    stage_us /= args.steps
    dense_stage = None
    if not args.no_dense:
        devs = [[pq.HipEvent() for _ in range(3)] for _ in range(args.steps)]
        for i in range(args.steps):
            L_ = layers[i % n_layers]
            pq.decode_step_profiled(shape, None, q, L_["kc"], L_["vc"], L_["bt"], ctx, out,
                                    dense_ws, devs[i], dense=True)
        torch.cuda.synchronize()
        dense_stage = [float(np.mean([devs[i][s].elapsed_ms(devs[i][s + 1]) * 1e3
                                      for i in range(args.steps)])) for s in range(2)]
    log("stages µs: " + ", ".join(f"{n}={v:.2f}" for n, v in zip(pq.STAGE_NAMES, stage_us)))

    # exact rows and k per head from the last step's workspace
    lay = pq.workspace_layout(shape)
    BH = shape.batch * shape.num_kv_heads
    n_rows = ws[lay.n_rows:lay.n_rows + BH * 4].view(torch.int32).cpu().numpy()
    k_sel = np.array([min(-(-int(inp.context_lens[b]) * inp.budget_bp // 10000),
                          10 ** 9) for b in range(inp.batch) for _ in range(inp.num_kv_heads)])
    alg = algorithmic_bytes(inp, n_rows, k_sel)

    if args.copy_calibration:
        n = 1 << 28                                   # 1 GiB of fp32
        src = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: {n * 4} bytes read and written")

    # dominant kernel and its roofline over algorithmic bytes
    names = pq.STAGE_NAMES
    dom = int(np.argmax(stage_us))
    per_stage_bytes = {"tables": alg["tables"], "scan": alg["scan"], "collect": None,
                       "select": None, "attend": alg["exact"] + alg["background"], "merge": None}
    dom_bytes = per_stage_bytes[names[dom]]
    achieved = dom_bytes / (stage_us[dom] * 1e-6) / 1e9 if dom_bytes else None
    roofline = {"bound": "hbm", "kernel": names[dom], "achieved": achieved, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": (achieved / HBM_PEAK_GBS) if achieved else None,
                "traffic": None, "alg_bytes_per_launch": dom_bytes,
                "launch_us": float(stage_us[dom])}

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
               "host_threads_available": os.cpu_count()}
        log(f"oracle: {cpu['value'] / 1e3:.1f} ms/step on ~{cpu['cores']} cores")

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
        "dense_us": dense_ms * 1e3 if dense_ms else None,
        "speedup_vs_dense": (dense_ms / ms) if dense_ms else None,
        "step_alg_bytes": alg["total"],
        "step_alg_gbps": alg["total"] / (ms * 1e-3) / 1e9,
        "dense_alg_gbps": (kv_bytes / (dense_ms * 1e-3) / 1e9) if dense_ms else None,
        "stages_us": {n: float(v) for n, v in zip(names, stage_us)},
        "dense_stages_us": ({"splitk": dense_stage[0], "merge": dense_stage[1]}
                            if dense_stage else None),
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
