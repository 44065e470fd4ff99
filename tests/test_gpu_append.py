"""GPU parity of pqhsa_append_tokens (through the C ABI) against the append
oracle, and of a decode step on the appended index against the decode oracle.

Encoder decisions are taken in fp32 on the GPU and in float64 by the oracle;
a choice counts as correct when its distance is within the fp32 rounding
band of the exact minimum (several choices are then correct), otherwise it
must equal the oracle's.  Where every distance is exact in fp32 (dyadic
inputs), ties are exact too and the lower id must win on both sides.
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


from gpu_helpers import check_output, check_selection, log  # noqa: E402
from pqhsa_synth import make_step_inputs  # noqa: E402

BAND_REL = 2e-5     # fp32 sum of 128 (or 8) squared differences


def _f64(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _setup(inp):
    import ivf_pq_sparse_amd as pq
    from pqhsa_synth.device import stage
    tens, kw = stage(inp, "cuda")
    shape = pq.make_shape(**kw)
    dec = pq.PQHSADecoder(shape)
    dec.upload(tens["centroids"], tens["codebooks"], tens["list_ids"], tens["codes"],
               tens["n_indexed"], tens["v_cache"], tens["block_table"])
    return tens, shape, dec


def _check_encoding(inp, b, h, t0, t1, lists, codes, stride=1):
    from oracle import pqhsa_append as ap
    K = _f64(inp.k_bits[b, h, t0:t1])[::stride]
    lists, codes = lists[::stride], codes[::stride]
    C = inp.centroids[b, h].astype(np.float64)
    B = inp.codebooks[b, h].astype(np.float64)
    ol, oc = ap.encode_tokens(K, C, B)
    lg, cg, lmin, cmin = ap.distance_gaps(K, C, B, lists, codes)
    assert np.all(lg <= BAND_REL * lmin + 1e-6), "list outside the fp32 band"
    same_l = lists == ol
    # codes are only comparable where the list agrees
    cg = cg[same_l]
    assert np.all(cg <= BAND_REL * cmin[same_l] + 1e-6), "code outside the fp32 band"
    return int((~same_l).sum()), int((codes[same_l] != oc[same_l]).sum())


# the last two append more than one 4096-token placement tile, with many
# lists (16 and 3 counting chunks per tile); their encodings are checked on
# every 29th token, the placement of all of them
@pytest.mark.parametrize("G,Hkv,L,tail,T", [(4, 2, 64, 512, 6000), (8, 1, 128, 300, 6000),
                                             (1, 3, 40, 17, 6000), (4, 1, 2000, 9000, 12000),
                                             (2, 1, 8192, 5000, 9000),
                                             # one new token; a single list; one token short
                                             # of and one past a placement tile
                                             (2, 3, 7, 1, 3000), (4, 1, 1, 100, 2000),
                                             (8, 2, 33, 4095, 6000), (4, 2, 300, 4097, 8000)])
def test_append_tail_matches_oracle(G, Hkv, L, tail, T):
    from oracle import pqhsa_append as ap
    from oracle import pqhsa_oracle as orc
    import oracle
    inp = make_step_inputs(1, context_lens=[T, T - 1111], batch=2, num_q_heads=G * Hkv,
                           num_kv_heads=Hkv, num_lists=L, n_tail=tail, budget_bp=150,
                           workload_id=300 + G)
    tens, shape, dec = _setup(inp)
    old = inp.n_indexed.copy()
    lay = __import__("ivf_pq_sparse_amd").index_layout(shape)
    cap = shape.max_context
    means_old = dec.index[lay.means:lay.means + 2 * Hkv * L * 512].view(torch.float32).clone()
    # forget the tail's generating lists and codes: the encoder must write them
    for b in range(2):
        tens["list_ids"][b, :, old[b]:] = -7
        tens["codes"][b, :, old[b]:] = 0
    new_n = torch.tensor(inp.context_lens, dtype=torch.int32, device="cuda")
    log(f"[append] G={G} Hkv={Hkv} L={L} tail={tail}")
    dec.append(tens["k_cache"], tens["v_cache"], tens["block_table"], new_n, tail,
               tens["list_ids"], tens["codes"])
    torch.cuda.synchronize()
    gl = tens["list_ids"].cpu().numpy()
    gc = tens["codes"].cpu().numpy().astype(np.int64)
    off = dec.index[lay.list_off:lay.list_off + 2 * Hkv * (L + 1) * 4].view(torch.int32)
    off = off.cpu().numpy().reshape(2, Hkv, L + 1)
    pos = dec.index[lay.pos:lay.pos + 2 * Hkv * cap * 4].view(torch.int32).cpu().numpy()
    pos = pos.reshape(2, Hkv, cap)
    mu = dec.index[lay.means:lay.means + 2 * Hkv * L * 512].view(torch.float32).cpu().numpy()
    mu = mu.reshape(2, Hkv, L, 128).astype(np.float64)
    mu_old = means_old.cpu().numpy().reshape(2, Hkv, L, 128).astype(np.float64)
    n_idx = dec.index[lay.n_indexed:lay.n_indexed + 8].view(torch.int32).cpu().numpy()
    assert list(n_idx) == list(inp.context_lens)
    diff_l = diff_c = 0
    for b in range(2):
        T_b = int(inp.context_lens[b])
        for h in range(Hkv):
            dl, dc = _check_encoding(inp, b, h, old[b], T_b, gl[b, h, old[b]:T_b],
                                     gc[b, h, old[b]:T_b], stride=29 if L > 1000 else 1)
            diff_l += dl
            diff_c += dc
            # regrouped index: cluster sizes and token order inside clusters
            allists = gl[b, h, :T_b]
            assert np.array_equal(np.diff(off[b, h]), np.bincount(allists, minlength=L))
            for c in range(L):
                pc = pos[b, h, off[b, h, c]:off[b, h, c + 1]]
                assert np.array_equal(pc, np.nonzero(allists == c)[0]), (b, h, c)
            # incremental means against the oracle's update of the GPU's old means
            n_old = np.bincount(inp.list_ids[b, h, :old[b]], minlength=L)
            ref, _ = ap.append_means(mu_old[b, h], n_old,
                                     orc.bf16_to_f64(inp.v_bits[b, h, old[b]:T_b]),
                                     gl[b, h, old[b]:T_b], L)
            np.testing.assert_allclose(mu[b, h], ref, atol=3e-6)
            # and the means of all members at once
            batch = orc.cluster_means(orc.bf16_to_f64(inp.v_bits[b, h, :T_b]), allists, L)
            np.testing.assert_allclose(mu[b, h], batch, atol=3e-6)
    log(f"[append] near-tie differences: lists {diff_l}, codes {diff_c}")
    # a decode step on the appended index against the oracle on the same state
    inp2 = inp
    inp2.list_ids = gl.copy()
    inp2.codes = gc.astype(np.uint8)
    inp2.n_indexed = inp.context_lens.copy()
    out, sel, lse = dec.step(tens["q"], tens["k_cache"], tens["v_cache"], tens["block_table"],
                             tens["context_lens"], selected=True, lse=True)
    torch.cuda.synchronize()
    assert dec.flags() == 0
    from gpu_helpers import oracle_with_details
    ref = oracle_with_details(inp2)
    s = sel.cpu().numpy()
    gsel = {(b, h): s[b, h][s[b, h] >= 0].astype(np.int64) for b in range(2) for h in range(Hkv)}
    check_selection(gsel, ref)
    again = oracle.decode_step(inp2, selected=gsel)
    check_output(out.cpu().numpy().astype(np.float64), again["O"], "decode after append")


def test_append_nothing_changes_nothing():
    inp = make_step_inputs(1, context_lens=[3000], num_q_heads=8, num_kv_heads=2, num_lists=32,
                           n_tail=200, workload_id=320)
    tens, shape, dec = _setup(inp)
    before = dec.index.clone()
    new_n = torch.tensor(inp.n_indexed, dtype=torch.int32, device="cuda")
    dec.append(tens["k_cache"], tens["v_cache"], tens["block_table"], new_n, 0,
               tens["list_ids"], tens["codes"])
    torch.cuda.synchronize()
    assert torch.equal(before, dec.index)


def test_append_into_an_empty_index():
    from oracle import pqhsa_oracle as orc
    inp = make_step_inputs(1, context_lens=[2500], num_q_heads=4, num_kv_heads=1, num_lists=16,
                           n_tail=2500, workload_id=321)
    tens, shape, dec = _setup(inp)
    new_n = torch.tensor(inp.context_lens, dtype=torch.int32, device="cuda")
    dec.append(tens["k_cache"], tens["v_cache"], tens["block_table"], new_n, 2500,
               tens["list_ids"], tens["codes"])
    torch.cuda.synchronize()
    import ivf_pq_sparse_amd as pq
    lay = pq.index_layout(shape)
    gl = tens["list_ids"].cpu().numpy()[0, 0, :2500]
    gc = tens["codes"].cpu().numpy()[0, 0, :2500].astype(np.int64)
    _check_encoding(inp, 0, 0, 0, 2500, gl, gc)
    mu = dec.index[lay.means:lay.means + 16 * 512].view(torch.float32).cpu().numpy()
    batch = orc.cluster_means(orc.bf16_to_f64(inp.v_bits[0, 0, :2500]), gl, 16)
    np.testing.assert_allclose(mu.reshape(16, 128), batch, atol=3e-6)


def test_append_exact_ties_take_lower_ids():
    # Dyadic centroids and codewords with noise-free keys make every fp32
    # distance exact; a centroid copied over a higher-numbered one and a
    # codeword copied over a higher-numbered one make exact ties.  The
    # encoder must take the lower list and the lower codeword every time, and
    # so equal the oracle token for token.
    from oracle import pqhsa_append as ap
    L, tail, T = 16, 600, 3000
    inp = make_step_inputs(1, context_lens=[T], num_q_heads=4, num_kv_heads=1, num_lists=L,
                           n_tail=tail, dyadic=True, noise=0.0, workload_id=322)
    old = int(inp.n_indexed[0])
    lists_tail = inp.list_ids[0, 0, old:T]
    a = int(np.bincount(lists_tail, minlength=L).argmax())     # a list with many new tokens
    b = L - 1 if a != L - 1 else L - 2
    assert a < b
    inp.centroids[0, 0, b] = inp.centroids[0, 0, a]
    m = 5
    codes_m = inp.codes[0, 0, old:T, m][lists_tail == a]
    j1 = int(np.bincount(codes_m, minlength=256).argmax())
    j2 = 255 if j1 != 255 else 254
    assert j1 < j2
    inp.codebooks[0, 0, m, j2] = inp.codebooks[0, 0, m, j1]
    tens, shape, dec = _setup(inp)
    tens["list_ids"][0, :, old:] = -7
    tens["codes"][0, :, old:] = 0
    new_n = torch.tensor([T], dtype=torch.int32, device="cuda")
    log(f"[append] planted ties: lists {a}/{b}, subspace {m} codewords {j1}/{j2}")
    dec.append(tens["k_cache"], tens["v_cache"], tens["block_table"], new_n, tail,
               tens["list_ids"], tens["codes"])
    torch.cuda.synchronize()
    gl = tens["list_ids"].cpu().numpy()[0, 0, old:T]
    gc = tens["codes"].cpu().numpy()[0, 0, old:T].astype(np.int64)
    K = _f64(inp.k_bits[0, 0, old:T])
    ol, oc = ap.encode_tokens(K, inp.centroids[0, 0].astype(np.float64),
                              inp.codebooks[0, 0].astype(np.float64))
    n_tied_l = int((lists_tail == a).sum())
    n_tied_c = int(((lists_tail == a) & (inp.codes[0, 0, old:T, m] == j1)).sum())
    assert n_tied_l > 0 and n_tied_c > 0
    assert not np.any(gl == b), "an exact list tie went to the higher list"
    assert not np.any(gc[:, m] == j2), "an exact codeword tie went to the higher codeword"
    assert np.array_equal(gl, ol) and np.array_equal(gc, oc)
    log(f"[append] {n_tied_l} list ties and {n_tied_c} codeword ties, all to the lower id")


def test_append_more_tokens_than_max_new():
    # max_new bounds every sequence's append: only that many tokens join the
    # index, the rest stay in the exact tail (unencoded), and a decode step on
    # the result matches the oracle with that shorter index
    import ivf_pq_sparse_amd as pq
    import oracle
    from gpu_helpers import oracle_with_details
    inp = make_step_inputs(1, context_lens=[4000, 3500], batch=2, num_q_heads=8, num_kv_heads=2,
                           num_lists=32, n_tail=300, budget_bp=150, workload_id=323)
    tens, shape, dec = _setup(inp)
    old = inp.n_indexed.copy()
    for b in range(2):
        tens["list_ids"][b, :, old[b]:] = -7
    max_new = 100
    new_n = torch.tensor(inp.context_lens, dtype=torch.int32, device="cuda")
    log("[append] 300 new tokens per sequence requested, max_new 100")
    dec.append(tens["k_cache"], tens["v_cache"], tens["block_table"], new_n, max_new,
               tens["list_ids"], tens["codes"])
    torch.cuda.synchronize()
    lay = pq.index_layout(shape)
    n_idx = dec.index[lay.n_indexed:lay.n_indexed + 8].view(torch.int32).cpu().numpy()
    assert list(n_idx) == [int(o) + max_new for o in old]
    gl = tens["list_ids"].cpu().numpy()
    gc = tens["codes"].cpu().numpy()
    for b in range(2):
        assert np.all(gl[b, :, old[b]:old[b] + max_new] >= 0)
        assert np.all(gl[b, :, old[b] + max_new:inp.context_lens[b]] == -7)
    L = shape.num_lists
    off = dec.index[lay.list_off:lay.list_off + 2 * 2 * (L + 1) * 4].view(torch.int32)
    off = off.cpu().numpy().reshape(2, 2, L + 1)
    assert np.all(off[:, :, L] == (old + max_new)[:, None])
    inp.n_indexed = (old + max_new).astype(np.int32)
    for b in range(2):
        n = int(inp.n_indexed[b])
        inp.list_ids[b, :, :n] = gl[b, :, :n]
        inp.codes[b, :, :n] = gc[b, :, :n]
    out, sel, lse = dec.step(tens["q"], tens["k_cache"], tens["v_cache"], tens["block_table"],
                             tens["context_lens"], selected=True, lse=True)
    torch.cuda.synchronize()
    assert dec.flags() == 0
    ref = oracle_with_details(inp)
    s = sel.cpu().numpy()
    gsel = {(b, h): s[b, h][s[b, h] >= 0].astype(np.int64) for b in range(2) for h in range(2)}
    check_selection(gsel, ref)
    again = oracle.decode_step(inp, selected=gsel)
    check_output(out.cpu().numpy().astype(np.float64), again["O"], "decode after a capped append")
