"""pqhsa_decode_step_noalloc (the decode step on the library's fixed
per-device scratch) against pqhsa_decode_step on the same inputs, through the
C ABI: identical selections, outputs and log-sum-exp, on two calls in a row
(the second smaller, in another layout of the scratch), each also checked
against the oracle.  (A shape too large for the scratch is refused before
anything is launched; the CPU ABI tests cover that.)"""
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


from gpu_helpers import check_result, log  # noqa: E402
from pqhsa_synth import make_step_inputs  # noqa: E402


def _both(inp, staged_expected=False):
    """Run the workspace entry point and the no-alloc one on the same index;
    return both results."""
    import ivf_pq_sparse_amd as pq
    from pqhsa_synth.device import stage
    tens, kw = stage(inp, "cuda")
    shape = pq.make_shape(**kw)
    dec = pq.PQHSADecoder(shape)
    dec.upload(tens["centroids"], tens["codebooks"], tens["list_ids"], tens["codes"],
               tens["n_indexed"], tens["v_cache"], tens["block_table"])
    args = (tens["q"], tens["k_cache"], tens["v_cache"], tens["block_table"], tens["context_lens"])
    o1, s1, l1 = dec.step(*args, selected=True, lse=True)
    B, Hq, Hkv = shape.batch, shape.num_q_heads, shape.num_kv_heads
    o2 = torch.full((B, Hq, 128), float("nan"), device="cuda")
    l2 = torch.full((B, Hq), float("nan"), device="cuda")
    s2 = torch.full_like(s1, -7)
    pq.decode_step_noalloc(shape, dec.index, *args, o2, selected=s2, lse=l2)
    torch.cuda.synchronize()
    assert dec.flags() == 0
    return shape, (o1, s1, l1), (o2, s2, l2)


def _compare(inp, what):
    shape, (o1, s1, l1), (o2, s2, l2) = _both(inp)
    # same kernels on the same inputs: the selection is bit-exact, and so are
    # the outputs (the step is deterministic)
    assert torch.equal(s1, s2), f"{what}: selections differ"
    assert torch.equal(o1, o2), f"{what}: outputs differ (max {float((o1 - o2).abs().max())})"
    assert torch.equal(l1, l2), f"{what}: lse differs"
    # and the no-alloc result meets the oracle bar by itself
    s = s2.cpu().numpy()
    g = dict(O=o2.cpu().numpy().astype(np.float64), lse=l2.cpu().numpy(),
             selected={(b, h): s[b, h][s[b, h] >= 0].astype(np.int64)
                       for b in range(shape.batch) for h in range(shape.num_kv_heads)})
    check_result(g, inp, what=f"{what} (no-alloc)")
    log(f"[noalloc] {what}: identical to the workspace entry point")


def test_noalloc_matches_workspace_entry_twice_second_smaller():
    _compare(make_step_inputs(1), "32K, 32q/8kv, L256")
    _compare(make_step_inputs(1, context_lens=[3000, 1711, 2222], batch=3, num_q_heads=8,
                              num_kv_heads=2, num_lists=24, n_tail=50, budget_bp=300,
                              workload_id=71), "ragged batch of 3, 8q/2kv, L24")


def test_noalloc_staged_shape():
    # 320 KV heads exceed what the device holds at once: the staged kernels
    # run on the scratch
    lens = [500 + 13 * b for b in range(40)]
    _compare(make_step_inputs(1, context_lens=lens, batch=40, num_q_heads=32, num_kv_heads=8,
                              num_lists=16, n_tail=40, budget_bp=500, workload_id=72),
             "40 sequences x 8 KV heads (staged)")
