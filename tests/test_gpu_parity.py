"""GPU parity of the HIP path (through the C ABI) against the float64 oracle."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import ivf_pq_sparse_amd as pq
    pq.load()          # raises if the HIP library is not built: no fallback


from gpu_helpers import (check_output, check_result, log, oracle_with_details,  # noqa: E402
                         parity, run_gpu)
from key_codes import key_code16  # noqa: E402
from pqhsa_synth import make_step_inputs  # noqa: E402


# ------------------------------------------------------------------ dense baseline
@pytest.mark.parametrize("T,G,Hkv", [(8192, 4, 1), (1000, 4, 2), (37, 8, 1), (5000, 1, 3),
                                     (2049, 2, 2), (3000, 2, 8), (4100, 4, 4), (700, 1, 6),
                                     (20000, 2, 1)])
def test_dense_matches_oracle(T, G, Hkv):
    import oracle
    inp = make_step_inputs(0, context_lens=[T], num_q_heads=G * Hkv, num_kv_heads=Hkv,
                           num_lists=8, workload_id=500 + T)
    log(f"[dense] T={T} G={G} Hkv={Hkv}")
    g = run_gpu(inp, dense=True)
    ref = oracle.dense_step(inp)
    check_output(g["O"], ref, f"dense T={T}")


@pytest.mark.parametrize("wid", [2, 4])
def test_dense_full_size_matches_oracle(wid):
    # the dense split-K step at the 128K and 512K layer shapes, in the launch
    # configuration the benchmark times, every query head against the oracle
    import oracle
    inp = make_step_inputs(wid)
    log(f"[dense] workload {wid} full size")
    g = run_gpu(inp, dense=True)
    check_output(g["O"], oracle.dense_step(inp), f"dense workload {wid}")


def test_dense_variable_lengths_and_spare_pages():
    import oracle
    inp = make_step_inputs(1, context_lens=[3000, 17, 1024, 2500], batch=4, num_q_heads=8,
                           num_kv_heads=2, num_lists=16, workload_id=77)
    log("[dense] ragged batch")
    g = run_gpu(inp, dense=True, spare_pages=9, page_seed=3, max_context=3100)
    check_output(g["O"], oracle.dense_step(inp), "dense ragged")


# ------------------------------------------------------------------ PQ-HSA step
def test_tiny_workload_parity():
    parity(make_step_inputs(0), what="workload 0 (8K, 4q/1kv, L64)")


def test_llama_32k_parity():
    parity(make_step_inputs(1), what="workload 1 (32K, 32q/8kv, L256)")


# Full-size workloads in the launch configuration bench.py times (same shape
# fields, so the same grids): every head at 128K, at 512K and of the
# 16-sequence batch, each head checked against the oracle in full.
def test_llama_128k_parity():
    parity(make_step_inputs(2), what="workload 2 (128K, 32q/8kv, L512, k=1311)")


@pytest.fixture(scope="module")
def batch16_run():
    """One GPU step of the 16-sequence batch (two fused blocks per head, the
    scan's cluster-claim path), shared by the four checks below."""
    inp = make_step_inputs(3)
    log("[parity] workload 3 (16 x 128K, 32q/8kv, L512): one GPU step")
    return inp, run_gpu(inp)


@pytest.mark.parametrize("part", range(4))
def test_llama_128k_batch16_parity(batch16_run, part):
    # every (sequence, KV head) of the batch, four sequences per test
    inp, g = batch16_run
    heads = [(b, h) for b in range(4 * part, 4 * part + 4) for h in range(inp.num_kv_heads)]
    check_result(g, inp, heads=heads,
                 what=f"workload 3 (16 x 128K), sequences {4 * part}..{4 * part + 3}, all KV heads")


def test_qwen_512k_parity():
    parity(make_step_inputs(4), what="workload 4 (512K, 32q/4kv G=8, L1024, k=5243)")


# Background term off (plain top-k sparse attention over sink, selected and
# recent tokens): the comparison of the PQ-HSA page's section B.
@pytest.mark.parametrize("staged", [False, True])
def test_exact_only_matches_oracle(staged):
    parity(make_step_inputs(1), what="workload 1, no background", staged=staged,
           background=False)


def test_exact_only_full_budget_is_dense():
    import oracle
    inp = make_step_inputs(1, context_lens=[4100], budget_bp=10000, num_lists=32, workload_id=9)
    g = run_gpu(inp, background=False)
    check_output(g["O"], oracle.dense_step(inp), "exact-only budget 100% vs dense")


def test_full_budget_is_dense_on_gpu():
    import oracle
    inp = make_step_inputs(1, context_lens=[4100], budget_bp=10000, num_lists=32, workload_id=9)
    log("[pqhsa] budget 100 %")
    g = run_gpu(inp)
    check_output(g["O"], oracle.dense_step(inp), "budget 100% vs dense")
    parity(inp, what="budget 100 %")


def test_budget_zero():
    inp = make_step_inputs(0, context_lens=[3000], budget_bp=0, num_lists=16, workload_id=10)
    g, _, _ = parity(inp, what="budget 0")
    assert all(v.size == 0 for v in g["selected"].values())


def test_one_token_clusters_zero_noise_equal_dense():
    import oracle
    T = 2048
    inp = make_step_inputs(0, context_lens=[T], dyadic=True, num_lists=T, one_token_per_list=True,
                           budget_bp=100, workload_id=11)
    log("[pqhsa] one token per cluster, zero noise")
    g = run_gpu(inp)
    check_output(g["O"], oracle.dense_step(inp), "one-token clusters vs dense")


def test_exact_ties_pick_lower_positions():
    # copy one candidate's (list, codes) over many others: their keys tie exactly
    inp = make_step_inputs(0, context_lens=[2000], num_lists=16, budget_bp=100, workload_id=12,
                           noise=0.0)
    ref = oracle_with_details(inp)
    kap, cand = ref["kappa"][(0, 0)], ref["candidates"][(0, 0)]
    src = int(cand[np.argmax(kap[cand])])
    dups = np.arange(100, 1900, 37)
    dups = dups[dups != src]
    inp.list_ids[0, 0, dups] = inp.list_ids[0, 0, src]
    inp.codes[0, 0, dups] = inp.codes[0, 0, src]
    g, ref, _ = parity(inp, what="exact ties")
    k = ref["k"][(0, 0)]
    tied = np.sort(np.concatenate([dups, [src]]))
    assert k < tied.size
    assert g["selected"][(0, 0)].tolist() == tied[:k].tolist()


def test_recent_longer_than_tail_and_ragged_batch():
    inp = make_step_inputs(1, context_lens=[5000, 3333, 777, 4096], batch=4, num_q_heads=8,
                           num_kv_heads=2, num_lists=64, n_tail=40, n_recent=200, n_sink=7,
                           budget_bp=250, workload_id=13)
    parity(inp, what="recent > tail, ragged batch", max_context=5003, page_seed=5)


def test_everything_forced_and_nothing_indexed():
    # sink + recent cover the context; and a sequence with no indexed token
    inp = make_step_inputs(1, context_lens=[300, 500], batch=2, num_q_heads=4, num_kv_heads=1,
                           num_lists=8, n_sink=100, n_recent=250, n_tail=0, budget_bp=500,
                           workload_id=14)
    parity(inp, what="all forced")
    inp2 = make_step_inputs(1, context_lens=[700], num_q_heads=4, num_kv_heads=1, num_lists=8,
                            n_tail=700, budget_bp=100, workload_id=15)
    g, _, _ = parity(inp2, what="empty index")
    assert g["selected"][(0, 0)].size == 0


def test_empty_and_one_token_sequences():
    # a sequence of length 0 attends to nothing (O = 0, lse = -inf); one of
    # length 1 attends to its only token
    inp = make_step_inputs(1, context_lens=[0, 1, 300], batch=3, num_q_heads=4, num_kv_heads=1,
                           num_lists=8, n_tail=0, budget_bp=500, workload_id=16)
    g, _, _ = parity(inp, what="lengths 0, 1 and 300")
    assert np.all(g["O"][0] == 0.0) and np.all(np.isneginf(g["lse"][0]))
    assert g["selected"][(0, 0)].size == 0 and g["selected"][(1, 0)].size == 0


def test_gqa_group_sizes():
    for G, Hkv in [(1, 4), (2, 2), (8, 1)]:
        inp = make_step_inputs(1, context_lens=[6000], num_q_heads=G * Hkv, num_kv_heads=Hkv,
                               num_lists=48, budget_bp=150, workload_id=20 + G)
        parity(inp, what=f"G={G}")


def test_index_means_match_oracle():
    import ivf_pq_sparse_amd as pq
    from oracle import pqhsa_oracle as orc
    inp = make_step_inputs(1, context_lens=[3000, 2000], batch=2, num_q_heads=8, num_kv_heads=2,
                           num_lists=40, workload_id=30)
    g = run_gpu(inp)
    shape, dec = g["shape"], g["dec"]
    lay = pq.index_layout(shape)
    L = shape.num_lists
    buf = dec.index
    means = buf[lay.means:lay.means + 2 * 2 * L * 128 * 4].view(torch.float32).cpu().numpy()
    means = means.reshape(2, 2, L, 128)
    off = buf[lay.list_off:lay.list_off + 2 * 2 * (L + 1) * 4].view(torch.int32).cpu().numpy()
    off = off.reshape(2, 2, L + 1)
    for b in range(2):
        Ti = int(inp.n_indexed[b])
        for h in range(2):
            mu = orc.cluster_means(orc.bf16_to_f64(inp.v_bits[b, h, :Ti]), inp.list_ids[b, h, :Ti], L)
            np.testing.assert_allclose(means[b, h], mu, atol=2e-6, rtol=1e-5)
            counts = np.bincount(inp.list_ids[b, h, :Ti], minlength=L)
            assert off[b, h, 0] == 0 and np.array_equal(np.diff(off[b, h]), counts)
    assert pq.index_dropped(shape, buf) == 0


@pytest.mark.parametrize("staged", [True, False])
def test_tables_and_keys_match_oracle(staged):
    # the staged path keeps the lookup table in the workspace; both paths keep
    # the centroid terms and the keys
    import ivf_pq_sparse_amd as pq
    from oracle import pqhsa_oracle as orc
    inp = make_step_inputs(1, context_lens=[4000], num_q_heads=8, num_kv_heads=2, num_lists=24,
                           workload_id=31)
    # the fused step passes its keys to its selection in LDS; the keys-out
    # variant also writes them to the workspace
    g = run_gpu(inp, staged=staged, variant=None if staged else pq.VARIANT_KEYS_OUT)
    shape, dec = g["shape"], g["dec"]
    lay = pq.workspace_layout(shape)
    ws = dec.workspace
    G, H, L = 4, 2, 24
    lut = ws[lay.lut:lay.lut + H * 16 * 256 * G * 4].view(torch.float32).cpu().numpy()
    lut = lut.reshape(H, 16, 256, G)
    qc = ws[lay.qc:lay.qc + H * L * G * 4].view(torch.float32).cpu().numpy().reshape(H, L, G)
    cap = shape.max_context
    if staged:
        keys = ws[lay.keys:lay.keys + H * cap * 4].view(torch.int32).cpu().numpy().view(np.uint32)
    else:
        # the fused step keeps the top 16 bits of each key
        keys = ws[lay.keys:lay.keys + H * cap * 2].view(torch.int16).cpu().numpy().view(np.uint16)
    ilay = pq.index_layout(shape)
    pos = dec.index[ilay.pos:ilay.pos + H * cap * 4].view(torch.int32).cpu().numpy()
    log2e = 1.0 / np.log(2.0)
    Ti = int(inp.n_indexed[0])
    F, Cand = orc.partition(int(inp.context_lens[0]), Ti, inp.n_sink, inp.n_recent)
    for h in range(H):
        q = orc.bf16_to_f64(inp.q_bits[0, h * G:(h + 1) * G])
        qc_ref, lut_ref = orc.lut_tables(q, inp.centroids[0, h].astype(np.float64),
                                         inp.codebooks[0, h].astype(np.float64), inp.scale)
        if staged:
            np.testing.assert_allclose(lut[h], np.transpose(lut_ref, (1, 2, 0)) * log2e,
                                       atol=2e-6)
        np.testing.assert_allclose(qc[h], qc_ref.T * log2e, atol=5e-6)
        # keys: order-preserving bits of max_g s_hat * log2e, 0 for non-candidates
        s = orc.approx_logits(qc_ref, lut_ref, inp.list_ids[0, h, :Ti], inp.codes[0, h, :Ti])
        kap = s.max(axis=0) * log2e
        p = pos[h * cap:h * cap + Ti]
        u = keys[h * cap:h * cap + Ti]
        iscand = np.isin(p, Cand)
        assert np.all(u[~iscand] == 0)
        f = u[iscand]
        if staged:
            bits = np.where(f & 0x80000000, f & 0x7FFFFFFF, ~f).astype(np.uint32)
            got = bits.view(np.float32).astype(np.float64)
            np.testing.assert_allclose(got, kap[p[iscand]], atol=2e-5, rtol=2e-6)
        else:
            # the 16-bit code of the fp32-rounded reference key: equal, or one
            # apart where fp32 rounding crosses a code boundary
            x = kap[p[iscand]].astype(np.float32).view(np.uint32)
            ref = key_code16(np.where(x & 0x80000000, ~x, x | 0x80000000).astype(np.uint32))
            assert np.all(f > 0)
            assert np.abs(f.astype(np.int64) - ref.astype(np.int64)).max() <= 1


def test_default_and_staged_paths_agree():
    # same tables in the same order: identical keys, so identical selections;
    # outputs differ only by summation order
    inp = make_step_inputs(2)
    log("[pqhsa] 128K: default vs staged")
    a = run_gpu(inp)
    b = run_gpu(inp, staged=True)
    for key in a["selected"]:
        assert np.array_equal(a["selected"][key], b["selected"][key]), key
    assert np.abs(a["O"] - b["O"]).max() < 2e-5
    assert np.abs(a["lse"] - b["lse"]).max() < 2e-5


def test_staged_kernels_match_oracle():
    parity(make_step_inputs(1), what="workload 1, staged kernels", staged=True)
    parity(make_step_inputs(4, context_lens=[70000], num_lists=256, workload_id=45),
           what="G=8 at 70K, staged kernels", staged=True)


def test_default_path_runs_one_kernel_on_the_workload_shapes():
    import ivf_pq_sparse_amd as pq
    from pqhsa_synth.device import stage
    for wid in (0, 1):
        inp = make_step_inputs(wid)
        tens, kw = stage(inp, "cuda")
        shape = pq.make_shape(**kw)
        dec = pq.PQHSADecoder(shape)
        dec.upload(tens["centroids"], tens["codebooks"], tens["list_ids"], tens["codes"],
                   tens["n_indexed"], tens["v_cache"], tens["block_table"])
        out = torch.empty(shape.batch, shape.num_q_heads, 128, device="cuda")
        evs = [pq.HipEvent() for _ in range(2 * pq.NUM_STAGES)]
        n = pq.decode_step_profiled(shape, dec.index, tens["q"], tens["k_cache"],
                                    tens["v_cache"], tens["block_table"], tens["context_lens"],
                                    out, dec.workspace, evs)
        torch.cuda.synchronize()
        assert n == 1, f"workload {wid}: {n} kernels"
        assert evs[0].elapsed_ms(evs[1]) > 0


def test_repeated_steps_are_deterministic():
    inp = make_step_inputs(1, context_lens=[20000], num_lists=128, workload_id=40)
    from pqhsa_synth.device import stage
    import ivf_pq_sparse_amd as pq
    tens, kw = stage(inp, "cuda")
    dec = pq.PQHSADecoder(pq.make_shape(**kw))
    dec.upload(tens["centroids"], tens["codebooks"], tens["list_ids"], tens["codes"],
               tens["n_indexed"], tens["v_cache"], tens["block_table"])
    first = None
    for _ in range(5):
        out, sel, _ = dec.step(tens["q"], tens["k_cache"], tens["v_cache"], tens["block_table"],
                               tens["context_lens"], selected=True)
        torch.cuda.synchronize()
        if first is None:
            first = (out.clone(), sel.clone())
        else:
            assert torch.equal(sel, first[1])
            assert torch.equal(out, first[0])


def test_tie_bucket_larger_than_the_lds_caches():
    # 90 % of the candidates copy the top candidate's list and codes: the
    # threshold bucket holds ~118K exact ties, more than the fused step's LDS
    # tie cache and, per block, more than its LDS staging of its own ties; the
    # winners are the lowest positions of the tie
    T = 131072
    inp = make_step_inputs(0, context_lens=[T], num_lists=64, budget_bp=100, noise=0.0,
                           workload_id=16)
    ref0 = oracle_with_details(inp)
    kap, cand = ref0["kappa"][(0, 0)], ref0["candidates"][(0, 0)]
    src = int(cand[np.argmax(kap[cand])])          # the largest key: the tie is the bucket
    rng = np.random.default_rng(16)
    dups = np.sort(rng.choice(cand[cand != src], size=int(0.9 * cand.size), replace=False))
    inp.list_ids[0, 0, dups] = inp.list_ids[0, 0, src]
    inp.codes[0, 0, dups] = inp.codes[0, 0, src]
    log("[pqhsa] 118K exact ties at 128K")
    g, ref, _ = parity(inp, what="huge tie bucket")
    sel = g["selected"][(0, 0)]
    tied = np.sort(np.concatenate([dups, [src]]))
    above = np.setdiff1d(sel, tied)
    k = ref["k"][(0, 0)]
    assert tied.size > 8192 and above.size == 0
    # the tied key is the largest: the selection is the tie's lowest positions
    assert np.array_equal(sel, tied[:k])


def test_full_budget_long_context_few_clusters():
    # 8 clusters over 64K tokens: 8 blocks of 8192 entries each, so the
    # selected-entry list and the attention item staging of a block both
    # overflow their LDS capacity and take their second paths
    import oracle
    inp = make_step_inputs(0, context_lens=[65536], num_lists=8, budget_bp=10000,
                           workload_id=17)
    log("[pqhsa] budget 100 % at 64K over 8 clusters")
    g = run_gpu(inp)
    check_output(g["O"], oracle.dense_step(inp), "budget 100% at 64K vs dense")
    parity(inp, what="budget 100 % at 64K, 8 clusters")


@pytest.mark.parametrize("G", [4, 8])
@pytest.mark.parametrize("budget_bp", [2500, 6000])
def test_many_key_chunks_per_block(budget_bp, G):
    # 2 clusters over 64K tokens: 2 blocks of 32K entries, four key chunks
    # each (8192 entries per chunk at G = 4, 9216 at G = 8).  At 25 % some
    # chunks' chosen entries fit the block's list and others are recorded
    # directly, so a listed chunk must be recorded before a later chunk is
    # recorded at the slots after it; at 60 % every chunk chooses more than
    # the list holds and records its own entries
    inp = make_step_inputs(0, context_lens=[65536], num_lists=2, budget_bp=budget_bp,
                           num_q_heads=G, num_kv_heads=1, workload_id=18)
    log(f"[pqhsa] budget {budget_bp} bp at 64K over 2 clusters, G={G}")
    parity(inp, what=f"budget {budget_bp} bp at 64K, 2 clusters, G={G}")


def _random_case(seed):
    """A seeded random shape: batch, heads, group size, ragged lengths
    (including empty and one-token sequences), list count, sink, recent
    window, tail, budget, background on or off, fused or staged path."""
    rng = np.random.default_rng([seed, 99])
    B = int(rng.integers(1, 4))
    Hkv = int(rng.integers(1, 4))
    G = int(rng.choice([1, 2, 4, 8]))
    lens = [int(rng.choice([0, 1, int(rng.integers(2, 7000))], p=[0.08, 0.07, 0.85]))
            for _ in range(B)]
    lens[0] = max(lens[0], int(rng.integers(1000, 7000)))
    kw = dict(batch=B, num_q_heads=G * Hkv, num_kv_heads=Hkv,
              num_lists=int(rng.choice([1, 3, 16, 64, 200, 700])),
              n_sink=int(rng.integers(0, 20)), n_recent=int(rng.integers(0, 300)),
              budget_bp=int(rng.choice([0, 1, 50, 100, 250, 1000, 5000, 10000])))
    tail = int(rng.integers(0, 400))
    background = bool(rng.random() < 0.75)
    staged = bool(rng.random() < 0.3)
    return lens, kw, tail, background, staged


@pytest.mark.parametrize("seed", range(32))
def test_random_shapes_match_oracle(seed):
    lens, kw, tail, background, staged = _random_case(seed)
    inp = make_step_inputs(1, context_lens=lens, n_tail=tail, workload_id=500 + seed, **kw)
    parity(inp, what=f"random case {seed}", page_seed=seed, staged=staged,
           background=background)


@pytest.mark.parametrize("B,expect_kernels", [(32, 1), (40, 6)])
def test_many_heads_one_block_each_or_staged(B, expect_kernels):
    # 32 sequences x 8 KV heads = 256 heads: the fused step runs one block per
    # head (no other block at its barriers); 40 x 8 = 320 heads exceed what
    # the device holds at once, so the default path is the staged kernels
    import ivf_pq_sparse_amd as pq
    from pqhsa_synth.device import stage
    lens = [600 + 37 * (b % 7) for b in range(B)]
    inp = make_step_inputs(1, context_lens=lens, batch=B, num_q_heads=32, num_kv_heads=8,
                           num_lists=16, n_tail=40, budget_bp=500, workload_id=40 + B)
    tens, kw = stage(inp, "cuda")
    shape = pq.make_shape(**kw)
    dec = pq.PQHSADecoder(shape)
    dec.upload(tens["centroids"], tens["codebooks"], tens["list_ids"], tens["codes"],
               tens["n_indexed"], tens["v_cache"], tens["block_table"])
    out = torch.empty(shape.batch, shape.num_q_heads, 128, device="cuda")
    evs = [pq.HipEvent() for _ in range(2 * pq.NUM_STAGES)]
    n = pq.decode_step_profiled(shape, dec.index, tens["q"], tens["k_cache"], tens["v_cache"],
                                tens["block_table"], tens["context_lens"], out, dec.workspace,
                                evs)
    torch.cuda.synchronize()
    assert n == expect_kernels
    parity(inp, what=f"{B} sequences x 8 KV heads")


def test_largest_list_count():
    # 16384 lists (the largest the library takes) over 40K tokens: about two
    # tokens per list, more lists per block than the fused step holds, so the
    # staged kernels run
    inp = make_step_inputs(1, context_lens=[40000], num_q_heads=8, num_kv_heads=2,
                           num_lists=16384, budget_bp=200, workload_id=52)
    parity(inp, what="16384 lists over 40K tokens")


@pytest.mark.parametrize("staged", [False, True])
def test_poisoned_workspace_parity(staged):
    # every scratch byte NaN (0xFF) before the step, counters and histogram
    # aside: a read of a partial, record or key the step did not write first
    # would reach the outputs
    parity(make_step_inputs(1), what="workload 1", staged=staged, poison=True)
    inp = make_step_inputs(1, context_lens=[5000, 3333, 777], batch=3, num_q_heads=16,
                           num_kv_heads=2, num_lists=64, n_tail=40, budget_bp=250,
                           workload_id=61)
    parity(inp, what="ragged batch", staged=staged, poison=True, page_seed=6)


@pytest.mark.parametrize("G", [4, 8])
def test_barrier_timeout_is_reported_and_cleared(G):
    # The barrier test variant waits for one block more than the grid has and
    # gives up after 20 us, so every wait runs out while every kernel still
    # ends normally: the call returns, the flag is set and every output is
    # NaN (at G = 8 through the tagged partials' timeout tag, elsewhere
    # through the head's flag).  After the flag is read and the workspace
    # cleared, the next step matches the oracle.
    import ivf_pq_sparse_amd as pq
    from pqhsa_synth.device import stage
    inp = make_step_inputs(1) if G == 4 else make_step_inputs(
        1, num_q_heads=32, num_kv_heads=4, workload_id=62)
    tens, kw = stage(inp, "cuda")
    shape = pq.make_shape(**kw)
    dec = pq.PQHSADecoder(shape)
    dec.upload(tens["centroids"], tens["codebooks"], tens["list_ids"], tens["codes"],
               tens["n_indexed"], tens["v_cache"], tens["block_table"])
    out = torch.zeros(shape.batch, shape.num_q_heads, 128, device="cuda")
    lse = torch.zeros(shape.batch, shape.num_q_heads, device="cuda")
    evs = [pq.HipEvent() for _ in range(2 * pq.NUM_STAGES)]
    log("[barrier] fused step with one phantom arrival per barrier")
    n = pq.decode_step_profiled(shape, dec.index, tens["q"], tens["k_cache"], tens["v_cache"],
                                tens["block_table"], tens["context_lens"], out, dec.workspace,
                                evs, variant=pq.VARIANT_BARRIER_TEST, lse=lse)
    torch.cuda.synchronize()
    assert n == 1
    assert torch.isnan(out).all() and torch.isnan(lse).all()
    assert dec.flags(clear=True) & 1
    assert dec.flags() == 0
    out2, sel, lse2 = dec.step(tens["q"], tens["k_cache"], tens["v_cache"], tens["block_table"],
                               tens["context_lens"], selected=True, lse=True)
    torch.cuda.synchronize()
    assert dec.flags() == 0
    s = sel.cpu().numpy()
    g = dict(O=out2.cpu().numpy().astype(np.float64), lse=lse2.cpu().numpy(),
             selected={(b, h): s[b, h][s[b, h] >= 0].astype(np.int64)
                       for b in range(shape.batch) for h in range(shape.num_kv_heads)})
    check_result(g, inp, what="step after a cleared barrier timeout")
