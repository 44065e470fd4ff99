"""Decode steps captured in a HIP graph (torch.cuda.graph) and replayed.

The steps leave their counters cleared by their own kernels (the fused step's
last block, the allocation-free entry point's fill kernel), never by a
memset, so a captured step can be replayed.  Each replay, with eager work and
synchronisations between replays, must give exactly the eager step's outputs
(the steps are deterministic), three steps per graph so that one captured
step runs on the counters the previous one left.
"""
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import ivf_pq_sparse_amd as pq
    pq.load()


from gpu_helpers import log  # noqa: E402
from pqhsa_synth import make_step_inputs  # noqa: E402


@pytest.mark.parametrize("kind", ["default", "noalloc", "dense"])
def test_graph_replays_match_eager_steps(kind):
    import ivf_pq_sparse_amd as pq
    from pqhsa_synth.device import stage
    inp = make_step_inputs(1, context_lens=[20000, 12000], batch=2, num_lists=128,
                           workload_id=41)
    tens, kw = stage(inp, "cuda")
    shape = pq.make_shape(**kw)
    dec = pq.PQHSADecoder(shape)
    dec.upload(tens["centroids"], tens["codebooks"], tens["list_ids"], tens["codes"],
               tens["n_indexed"], tens["v_cache"], tens["block_table"])
    dws = dec.dense_workspace()
    B, Hq = shape.batch, shape.num_q_heads
    n = 3

    def run(outs, lses):
        for o, ls in zip(outs, lses):
            args = (tens["q"], tens["k_cache"], tens["v_cache"], tens["block_table"],
                    tens["context_lens"], o)
            if kind == "default":
                pq.decode_step(shape, dec.index, *args, dec.workspace, lse=ls)
            elif kind == "noalloc":
                pq.decode_step_noalloc(shape, dec.index, *args, lse=ls)
            else:
                pq.dense_decode_step(shape, *args, dws, lse=ls)

    def buffers():
        return ([torch.empty(B, Hq, 128, dtype=torch.float32, device="cuda") for _ in range(n)],
                [torch.empty(B, Hq, dtype=torch.float32, device="cuda") for _ in range(n)])

    eo, el = buffers()
    run(eo, el)
    torch.cuda.synchronize()
    ref_o, ref_l = eo[0].clone(), el[0].clone()
    for o, ls in zip(eo, el):
        assert torch.equal(o, ref_o) and torch.equal(ls, ref_l)

    go, gl = buffers()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(go, gl)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(go, gl)
    log(f"[graph] {kind}: captured {n} steps")
    for rep in range(4):
        for o, ls in zip(go, gl):
            o.fill_(float("nan"))
            ls.fill_(float("nan"))
        # eager steps between the replays, on other output buffers
        run(eo, el)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (o, ls) in enumerate(zip(go, gl)):
            assert torch.equal(o, ref_o), f"{kind}: replay {rep} step {i} output differs"
            assert torch.equal(ls, ref_l), f"{kind}: replay {rep} step {i} lse differs"
    if kind == "default":
        assert dec.flags() == 0
