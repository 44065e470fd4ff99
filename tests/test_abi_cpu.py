"""Host-side checks of libpqhsa that need no GPU.

Every call here fails validation before anything is enqueued, so no kernel
is ever launched (the pointers passed are placeholders and must never be
dereferenced).
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pqhsa.h")

OK, INVALID, UNSUPPORTED, TOO_SMALL, HIP = 0, 1, 2, 3, 4


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pqhsa_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    from ivf_pq_sparse_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libpqhsa.so is not built (run __graft_entry__.build())")
    return _lib.load()


@pytest.fixture
def shape():
    from ivf_pq_sparse_amd import make_shape
    return make_shape(batch=1, num_q_heads=32, num_kv_heads=8, num_pages=8192,
                      max_pages_per_seq=8192, max_context=131072, num_lists=512, n_sink=4,
                      n_recent=128, budget_bp=100)


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 12
    from ivf_pq_sparse_amd import _lib
    assert sorted(_lib.EXPORTS) == names
    for n in names:
        assert hasattr(lib, n), f"{n} not exported"


def test_status_strings(lib):
    from ivf_pq_sparse_amd import status_string
    assert status_string(OK) == "ok"
    assert status_string(INVALID) == "invalid argument"
    assert status_string(UNSUPPORTED) == "unsupported shape"
    assert status_string(TOO_SMALL) == "buffer too small"
    assert status_string(HIP) == "HIP error"
    assert status_string(99) == "unknown status"


def test_sizes_for_the_128k_layer(shape):
    import ivf_pq_sparse_amd as pq
    assert pq.max_selected(shape) == 1311
    ib = pq.index_bytes(shape)
    # codes 16 B + position 4 B + cluster id 4 B per token and head,
    # centroids, means, codebooks
    BH, cap, L = 8, 131072, 512
    floor = BH * cap * 24 + BH * L * 128 * 4 * 2 + BH * 16 * 256 * 8 * 4
    assert floor <= ib <= floor + 64 * 1024
    ws = pq.workspace_bytes(shape)
    lay = pq.workspace_layout(shape)
    assert lay.n_parts == lay.n_exact_splits + lay.n_bg_splits
    assert lay.partials + 1 * 32 * lay.n_parts * 132 * 4 <= ws
    dws = pq.workspace_bytes(shape, dense=True)
    dl = pq.workspace_layout(shape, dense=True)
    # dense split-K: about 512 blocks in all, a multiple of 8 splits per head
    assert dl.n_bg_splits == 0 and dl.n_exact_splits == 64
    assert dws >= 32 * dl.n_parts * 132 * 4
    assert pq.upload_workspace_bytes(shape) >= BH * (cap // 4096) * L * 4


@pytest.mark.parametrize("field,value,expect", [
    ("batch", 0, INVALID), ("num_kv_heads", 0, INVALID), ("num_q_heads", 12, INVALID),
    ("num_q_heads", 8 * 16, UNSUPPORTED), ("head_dim", 64, UNSUPPORTED),
    ("page_size", 32, UNSUPPORTED), ("num_lists", 0, INVALID), ("num_lists", 20000, UNSUPPORTED),
    ("pq_m", 8, UNSUPPORTED), ("pq_ksub", 16, UNSUPPORTED), ("budget_bp", 10001, INVALID),
    ("budget_bp", -1, INVALID), ("n_sink", -1, INVALID), ("n_recent", -2, INVALID),
    ("max_context", 131072 + 17, INVALID), ("scale", 0.0, INVALID), ("scale", float("nan"), INVALID),
    ("num_pages", 0, INVALID), ("exact_only", 2, INVALID), ("exact_only", -1, INVALID),
])
def test_invalid_shapes_are_rejected(lib, shape, field, value, expect):
    import ivf_pq_sparse_amd as pq
    setattr(shape, field, value)
    assert pq.index_bytes(shape) == 0
    assert pq.workspace_bytes(shape) == 0
    fake = ctypes.c_void_p(0x1000)
    st = lib.pqhsa_decode_step(ctypes.byref(shape), fake, fake, fake, fake, fake, fake, fake,
                               None, None, fake, 1 << 40, None)
    assert st == expect
    st = lib.pqhsa_upload_index(ctypes.byref(shape), fake, fake, fake, fake, fake, fake, fake,
                                fake, 1 << 40, fake, 1 << 40, None)
    assert st == expect


def test_sparse_context_limit(lib, shape):
    import ivf_pq_sparse_amd as pq
    shape.max_pages_per_seq = 1 << 17
    shape.max_context = (1 << 20) + 16       # above the selection bitmap held in LDS
    assert pq.workspace_bytes(shape) == 0 and pq.index_bytes(shape) == 0
    assert pq.workspace_bytes(shape, dense=True) > 0     # the dense path has no such limit
    shape.max_context = 1 << 20
    assert pq.workspace_bytes(shape) > 0


def test_dense_ignores_method_fields(lib, shape):
    import ivf_pq_sparse_amd as pq
    shape.num_lists = 0
    shape.budget_bp = 99999
    assert pq.workspace_bytes(shape, dense=True) > 0
    assert pq.workspace_bytes(shape, dense=False) == 0


def test_null_pointers_and_small_buffers(lib, shape):
    fake = ctypes.c_void_p(0x1000)
    S = ctypes.byref(shape)
    # each required pointer missing in turn
    for i in range(7):
        args = [fake] * 7
        args[i] = None
        assert lib.pqhsa_decode_step(S, *args, None, None, fake, 1 << 40, None) == INVALID
    assert lib.pqhsa_decode_step(S, fake, fake, fake, fake, fake, fake, fake, None, None, None,
                                 1 << 40, None) == INVALID
    need = lib.pqhsa_workspace_bytes(S, 0)
    assert lib.pqhsa_decode_step(S, fake, fake, fake, fake, fake, fake, fake, None, None, fake,
                                 need - 1, None) == TOO_SMALL
    dneed = lib.pqhsa_workspace_bytes(S, 1)
    assert lib.pqhsa_dense_decode_step(S, fake, fake, fake, fake, fake, fake, None, fake,
                                       dneed - 1, None) == TOO_SMALL
    ineed = lib.pqhsa_index_bytes(S)
    assert lib.pqhsa_upload_index(S, fake, fake, fake, fake, fake, fake, fake, fake, ineed - 1,
                                  fake, 1 << 40, None) == TOO_SMALL
    uneed = lib.pqhsa_upload_workspace_bytes(S)
    assert lib.pqhsa_upload_index(S, fake, fake, fake, fake, fake, fake, fake, fake, ineed,
                                  fake, uneed - 1, None) == TOO_SMALL
    assert lib.pqhsa_decode_step_profiled(S, fake, fake, fake, fake, fake, fake, fake, None, None,
                                          fake, 1 << 40, 0, None, None, None) == INVALID
    # an unknown variant is rejected before anything is read or launched
    assert lib.pqhsa_decode_step_profiled(S, fake, fake, fake, fake, fake, fake, fake, None, None,
                                          fake, 1 << 40, 7, fake, None, None) == INVALID
    assert lib.pqhsa_index_dropped(S, None, None, None) == INVALID
    assert lib.pqhsa_workspace_layout(S, 0, None) == INVALID
    assert lib.pqhsa_index_layout_of(None, None) == INVALID


def test_noalloc_and_flags_validation(lib, shape):
    # the fixed-scratch step refuses a shape whose workspace exceeds the
    # scratch, and bad arguments, before it touches the device
    import ivf_pq_sparse_amd as pq
    fake = ctypes.c_void_p(0x1000)
    S = ctypes.byref(shape)
    assert pq.workspace_bytes(shape) <= pq.NOALLOC_SCRATCH_BYTES
    for i in range(7):
        args = [fake] * 7
        args[i] = None
        assert lib.pqhsa_decode_step_noalloc(S, *args, None, None, None) == INVALID
    big = pq.make_shape(batch=16, num_q_heads=32, num_kv_heads=8, num_pages=16 * 8192,
                        max_pages_per_seq=8192, max_context=131072, num_lists=512, n_sink=4,
                        n_recent=128, budget_bp=100)
    assert pq.workspace_bytes(big) > pq.NOALLOC_SCRATCH_BYTES
    assert lib.pqhsa_decode_step_noalloc(ctypes.byref(big), *([fake] * 7), None, None,
                                         None) == TOO_SMALL
    shape.budget_bp = -5
    assert lib.pqhsa_decode_step_noalloc(S, *([fake] * 7), None, None, None) == INVALID
    shape.budget_bp = 100
    flags = ctypes.c_uint32(0)
    need = lib.pqhsa_workspace_bytes(S, 0)
    assert lib.pqhsa_step_flags(S, None, need, 0, ctypes.byref(flags), None) == INVALID
    assert lib.pqhsa_step_flags(S, fake, need, 0, None, None) == INVALID
    assert lib.pqhsa_step_flags(S, fake, need - 1, 1, ctypes.byref(flags), None) == TOO_SMALL


def test_binding_rejects_cpu_tensors():
    torch = pytest.importorskip("torch")
    import ivf_pq_sparse_amd as pq
    from ivf_pq_sparse_amd import _lib
    with pytest.raises(ValueError):
        _lib._ptr(torch.zeros(4), "x", torch.float32)
    s = pq.make_shape(batch=1, num_q_heads=4, num_kv_heads=1, num_pages=4, max_pages_per_seq=4,
                      max_context=64, num_lists=4, budget_bp=100)
    with pytest.raises(ValueError):
        pq.dense_decode_step(s, torch.zeros(512, dtype=torch.int16), None, None, None, None,
                             None, None)


def test_reuse_sizes_window_limits_and_validation(lib, shape):
    import ivf_pq_sparse_amd as pq
    # rings: 32 heads x 1024 slots x (256 B search + 528 B state + 4 B context)
    # plus the counts: about 5 % of the layer's 512 MiB K/V cache at 128K
    nb = pq.reuse_buffer_bytes(shape, 1024)
    assert nb >= 32 * 1024 * (256 + 528 + 4) + 32 * 4
    assert 0.04 < nb / (131072 * 8 * 128 * 2 * 2) < 0.06
    lay = pq.reuse_layout(shape, 1024)
    assert lay.search == 0 and lay.states >= 32 * 1024 * 256
    assert lay.context >= lay.states + 32 * 1024 * 528 and lay.count > lay.context
    assert lay.total == nb
    assert pq.reuse_workspace_bytes(shape, 1024) > 0
    for w in (0, -1, 8193):
        assert pq.reuse_buffer_bytes(shape, w) == 0
        assert pq.reuse_workspace_bytes(shape, w) == 0
    assert pq.reuse_buffer_bytes(shape, 8192) > 0
    fake = ctypes.c_void_p(0x1000)
    S = ctypes.byref(shape)
    need = lib.pqhsa_reuse_buffer_bytes(S, 64)
    wneed = lib.pqhsa_reuse_workspace_bytes(S, 64)
    ok_args = [fake] * 7
    def call(window=64, thr=1.0, ptrs=None, nb=need, wb=wneed, buf=fake):
        p = ok_args if ptrs is None else ptrs
        return lib.pqhsa_reuse_decode_step(S, window, thr, p[0], p[1], p[2], p[3], p[4], p[5],
                                           buf, nb, p[6], None, None, None, fake, wb, None)
    for i in range(7):
        ptrs = list(ok_args)
        ptrs[i] = None
        assert call(ptrs=ptrs) == INVALID
    assert call(buf=None) == INVALID
    assert call(window=0) == INVALID and call(window=9000) == INVALID
    assert call(thr=float("nan")) == INVALID
    assert call(nb=need - 1) == TOO_SMALL
    assert call(wb=wneed - 1) == TOO_SMALL
    assert lib.pqhsa_reuse_decode_step_profiled(S, 64, 1.0, *ok_args[:6], fake, need, fake,
                                                None, None, None, fake, wneed, None, None,
                                                None) == INVALID
    assert lib.pqhsa_reuse_clear(S, 64, fake, need, 0, 2, None) == INVALID
    assert lib.pqhsa_reuse_clear(S, 64, fake, need, -1, 1, None) == INVALID
    assert lib.pqhsa_reuse_clear(S, 64, fake, need - 1, 0, 1, None) == TOO_SMALL
    assert lib.pqhsa_reuse_clear(S, 64, None, need, 0, 1, None) == INVALID
    assert lib.pqhsa_reuse_layout_of(S, 64, None) == INVALID
