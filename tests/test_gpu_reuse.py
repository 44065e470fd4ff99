"""GPU parity of the query-reuse decode step (through the C ABI) against the
query-reuse oracle, over streams of consecutive steps.

The reuse decision is taken in fp32 on the GPU and in float64 by the oracle:
a reported distance must lie within fp32 rounding of the exact minimum, and a
choice counts as correct when its exact distance is within that band of the
minimum (and of the threshold); the expected output is then computed by the
oracle with the GPU's choice.  Ring contents (context lengths, counts, search
vectors) must match exactly, stored states to the output tolerance.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import ivf_pq_sparse_amd as pq
    pq.load()


from gpu_helpers import LSE_ATOL, check_output, log  # noqa: E402
from pqhsa_synth import make_query_stream, make_step_inputs  # noqa: E402

BAND_REL = 2e-5     # fp32 sum of 128 squared differences


def _setup(B, Hq, Hkv, Tmax, wid, window, max_d2):
    import ivf_pq_sparse_amd as pq
    from pqhsa_synth.device import stage
    inp = make_step_inputs(1, context_lens=[Tmax] * B, batch=B, num_q_heads=Hq,
                           num_kv_heads=Hkv, num_lists=8, n_tail=0, n_planted=0,
                           workload_id=wid)
    tens, kw = stage(inp, "cuda")
    shape = pq.make_shape(**kw)
    dec = pq.ReuseDecoder(shape, window=window, max_dist2=max_d2)
    return inp, tens, shape, dec


def _check_decision(obuf, b, hq, x, T, max_d2, gslot, gd2):
    from oracle import pqhsa_reuse as ru
    cand = ru.eligible(obuf, b, hq, T)
    if cand.size == 0:
        assert gslot == -1 and np.isinf(gd2), (b, hq, gslot, gd2)
        return False
    d = ru.sq_dists(obuf, b, hq, x)
    dmin = d[cand].min()
    band = BAND_REL * dmin + 1e-6
    assert abs(gd2 - dmin) <= band, (b, hq, gd2, dmin)
    if gslot >= 0:
        assert gslot in cand, (b, hq, gslot)
        assert d[gslot] <= dmin + band, (b, hq, d[gslot], dmin)
        assert d[gslot] <= max_d2 + BAND_REL * abs(max_d2) + 1e-6
        return True
    assert dmin >= max_d2 - BAND_REL * abs(max_d2) - 1e-6, (b, hq, dmin, max_d2)
    return False


def _check_rings(dec, obuf, what):
    from oracle.pqhsa_oracle import bf16_to_f64
    ctx = dec.ring("context").cpu().numpy()
    cnt = dec.ring("count").cpu().numpy()
    assert np.array_equal(ctx, obuf.tj), f"{what}: ring context lengths"
    assert np.array_equal(cnt, obuf.cnt), f"{what}: ring counts"
    filled = ctx > 0
    qs = bf16_to_f64(dec.ring("search").cpu().numpy().view(np.uint16))
    assert np.array_equal(qs[filled], obuf.qs[filled]), f"{what}: ring search vectors"
    st = dec.ring("states").cpu().numpy().astype(np.float64)
    l = st[..., 1][filled]
    O_gpu = st[..., 4:][filled] / l[:, None]
    O_ref = obuf.N[filled] / obuf.Dn[filled][:, None]
    check_output(O_gpu, O_ref, f"{what}: stored states")
    lse_gpu = st[..., 0][filled] * np.log(2.0) + np.log(l)
    lse_ref = obuf.m[filled] + np.log(obuf.Dn[filled])
    assert np.abs(lse_gpu - lse_ref).max() <= LSE_ATOL, f"{what}: stored lse"


def _run_stream(B, Hq, Hkv, T0, incs, window, max_d2, wid, p_stay=0.7, jitter=0.05,
                separate_search=True):
    from oracle import pqhsa_reuse as ru
    from oracle.pqhsa_oracle import bf16_to_f64
    n = len(incs)
    Ts = np.array([[T0 + b * 37 + int(np.sum(incs[:i + 1])) for b in range(B)]
                   for i in range(n)])
    Tmax = int(Ts.max())
    inp, tens, shape, dec = _setup(B, Hq, Hkv, Tmax, wid, window, max_d2)
    q, qs, _ = make_query_stream(wid, B, Hq, n, p_stay=p_stay, jitter=jitter,
                                 separate_search=separate_search)
    obuf = ru.new_buffer(B, Hq, window)
    n_reuse = n_full = 0
    for i in range(n):
        log(f"[reuse] B={B} Hq={Hq} Hkv={Hkv} W={window} step {i} T={list(Ts[i])}")
        ctx = torch.tensor(Ts[i], dtype=torch.int32, device="cuda")
        qd = torch.from_numpy(q[i].view(np.int16)).cuda()
        qsd = torch.from_numpy(qs[i].view(np.int16)).cuda()
        out, lse, slot, d2 = dec.step(qd, qsd, tens["k_cache"], tens["v_cache"],
                                      tens["block_table"], ctx, lse=True, report=True)
        torch.cuda.synchronize()
        gslot = slot.cpu().numpy()
        gd2 = d2.cpu().numpy().astype(np.float64)
        xs = bf16_to_f64(qs[i])
        for b in range(B):
            for hq in range(Hq):
                used = _check_decision(obuf, b, hq, xs[b, hq], int(Ts[i, b]), max_d2,
                                       int(gslot[b, hq]), gd2[b, hq])
                n_reuse += used
                n_full += not used
        ref = ru.reuse_step(obuf, q[i], qs[i], inp.k_bits, inp.v_bits, Ts[i], inp.scale,
                            max_d2, choices=gslot)
        check_output(out.cpu().numpy().astype(np.float64), ref["O"], f"step {i}")
        lerr = np.abs(lse.cpu().numpy().astype(np.float64) - ref["lse"]).max()
        assert lerr <= LSE_ATOL, f"step {i}: lse error {lerr:.3e}"
    _check_rings(dec, obuf, "after the stream")
    log(f"[reuse] heads reused {n_reuse}, computed in full {n_full}")
    return dec, obuf, n_reuse, n_full


# increments of the context length between steps: repeats (T_j = T), single
# tokens, and jumps past the window
INCS = [0, 1, 1, 0, 1, 2, 1, 1, 1, 25, 1, 1, 3, 1, 1, 1, 0, 1, 1, 1, 40, 1, 1, 1]


@pytest.mark.parametrize("B,Hq,Hkv", [(2, 8, 2), (1, 4, 4), (2, 4, 2), (1, 16, 2)])
def test_reuse_stream_matches_oracle(B, Hq, Hkv):
    _, _, n_reuse, n_full = _run_stream(B, Hq, Hkv, 2900, INCS, window=16, max_d2=2.0,
                                        wid=400 + Hq + B)
    assert n_reuse > 0 and n_full > 0


def test_reuse_with_search_vector_equal_to_query():
    _run_stream(1, 8, 2, 1500, INCS[:12], window=8, max_d2=2.0, wid=420,
                separate_search=False)


def test_negative_threshold_never_reuses_and_equals_full_attention():
    _, _, n_reuse, _ = _run_stream(1, 8, 2, 1000, INCS[:8], window=16, max_d2=-1.0, wid=421)
    assert n_reuse == 0


def test_clear_empties_the_rings_of_chosen_sequences():
    import ivf_pq_sparse_amd as pq  # noqa: F401
    from oracle import pqhsa_reuse as ru
    dec, obuf, _, _ = _run_stream(2, 8, 2, 1200, INCS[:6], window=16, max_d2=2.0, wid=422)
    dec.clear(1, 2)
    torch.cuda.synchronize()
    obuf.tj[1] = 0
    obuf.cnt[1] = 0
    ctx = dec.ring("context").cpu().numpy()
    cnt = dec.ring("count").cpu().numpy()
    assert np.array_equal(ctx, obuf.tj) and np.array_equal(cnt, obuf.cnt)
    assert np.all(ru.eligible(obuf, 1, 0, 10 ** 6).size == 0)


def test_window_of_one_and_wide_window():
    _run_stream(1, 4, 1, 700, INCS[:10], window=1, max_d2=2.0, wid=423)
    _run_stream(1, 4, 1, 700, INCS[:10], window=300, max_d2=2.0, wid=424)


@pytest.mark.parametrize("seed", [0])
def test_full_size_llama_128k_stream(seed):
    # the 128K Llama-3.1-8B shape (32 query heads, 8 KV heads), the post's
    # 1024-token window, a few steps
    _, _, n_reuse, n_full = _run_stream(1, 32, 8, 131072 - 40, [0, 1, 1, 5, 1, 0, 1, 1],
                                        window=1024, max_d2=2.0, wid=430 + seed)
    assert n_reuse > 0 and n_full > 0
