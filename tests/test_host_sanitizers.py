"""The library's host logic (shape validation, buffer sizes and layouts:
ivf_pq_sparse_amd/csrc/pqhsa_host.cpp) built on its own with g++ under
AddressSanitizer and UndefinedBehaviorSanitizer, and driven through its C ABI
in a child process with valid, invalid and random shapes: every call must
return the documented status, every layout must be ordered, aligned and
inside its total, and neither sanitizer may report anything.  No GPU needed.
"""
import os
import shutil
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "ivf_pq_sparse_amd", "csrc")

# the ctypes structures of include/pqhsa.h, as the child process declares them
# (it does not import torch); checked against the package's own below
SHAPE_FIELDS = ["batch", "num_q_heads", "num_kv_heads", "head_dim", "page_size", "num_pages",
                "max_pages_per_seq", "num_lists", "pq_m", "pq_ksub", "max_context", "n_sink",
                "n_recent", "budget_bp", "scale", "exact_only"]
WS_FIELDS = ["lut", "qc", "keys", "bins", "rows", "n_rows", "partials", "flags",
             "n_exact_splits", "n_bg_splits", "n_parts", "hist", "hist_bytes", "counters",
             "counters_bytes", "total"]
INDEX_FIELDS = ["centroids", "codebooks", "list_off", "codes", "pos", "means", "n_indexed",
                "dropped"]
REUSE_FIELDS = ["search", "states", "context", "count", "total"]

DRIVER = textwrap.dedent(r'''
    import ctypes, math, random, sys
    lib = ctypes.CDLL(sys.argv[1])
    I32, SZ, F32 = ctypes.c_int32, ctypes.c_size_t, ctypes.c_float

    class Shape(ctypes.Structure):
        _fields_ = [(n, I32) for n in SHAPE_FIELDS[:-2]] + [("scale", F32), ("exact_only", I32)]

    class Ws(ctypes.Structure):
        _fields_ = [(n, SZ) for n in WS_FIELDS[:8]] + [(n, I32) for n in WS_FIELDS[8:11]] + [
            (n, SZ) for n in WS_FIELDS[11:]]

    class Ix(ctypes.Structure):
        _fields_ = [(n, SZ) for n in INDEX_FIELDS]

    class Ru(ctypes.Structure):
        _fields_ = [(n, SZ) for n in REUSE_FIELDS]

    P = ctypes.POINTER
    for name, res, args in [
            ("pqhsa_index_bytes", SZ, [P(Shape)]),
            ("pqhsa_upload_workspace_bytes", SZ, [P(Shape)]),
            ("pqhsa_workspace_bytes", SZ, [P(Shape), I32]),
            ("pqhsa_max_selected", I32, [P(Shape)]),
            ("pqhsa_append_workspace_bytes", SZ, [P(Shape)]),
            ("pqhsa_workspace_layout", I32, [P(Shape), I32, P(Ws)]),
            ("pqhsa_index_layout_of", I32, [P(Shape), P(Ix)]),
            ("pqhsa_reuse_buffer_bytes", SZ, [P(Shape), I32]),
            ("pqhsa_reuse_workspace_bytes", SZ, [P(Shape), I32]),
            ("pqhsa_reuse_layout_of", I32, [P(Shape), I32, P(Ru)]),
            ("pqhsa_status_string", ctypes.c_char_p, [I32])]:
        f = getattr(lib, name)
        f.restype, f.argtypes = res, args

    OK, INVALID, UNSUPPORTED = 0, 1, 2

    def shape(**kw):
        base = dict(batch=1, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16,
                    num_pages=512, max_pages_per_seq=512, num_lists=64, pq_m=16, pq_ksub=256,
                    max_context=8192, n_sink=4, n_recent=256, budget_bp=100, scale=0.088,
                    exact_only=0)
        base.update(kw)
        return Shape(**base)

    def check_offsets(offs, total, what):
        prev = -1
        for o in offs:
            assert o % 256 == 0, (what, offs)
            assert o >= prev, (what, offs)
            prev = o
        assert total >= prev and total % 256 == 0, (what, offs, total)

    def exercise(s):
        """Every sizing and layout call on one shape; returns the validity seen."""
        p = ctypes.byref(s)
        ok_sparse = lib.pqhsa_index_bytes(p) > 0
        assert (lib.pqhsa_upload_workspace_bytes(p) > 0) == ok_sparse
        assert (lib.pqhsa_append_workspace_bytes(p) > 0) == ok_sparse
        assert (lib.pqhsa_max_selected(p) >= 0)
        for dense in (0, 1):
            ws = Ws()
            st = lib.pqhsa_workspace_layout(p, dense, ctypes.byref(ws))
            nb = lib.pqhsa_workspace_bytes(p, dense)
            if st == OK:
                assert nb == ws.total > 0
                offs = [ws.partials] if dense else [ws.lut, ws.qc, ws.keys, ws.bins, ws.hist,
                                                    ws.rows, ws.n_rows, ws.counters, ws.flags,
                                                    ws.partials]
                check_offsets(sorted(offs), ws.total, "workspace")
                assert ws.n_parts == ws.n_exact_splits + ws.n_bg_splits >= 1
                if not dense:
                    assert ws.hist + ws.hist_bytes <= ws.total
                    assert ws.counters + ws.counters_bytes <= ws.total
            else:
                assert st in (INVALID, UNSUPPORTED) and nb == 0, (st, nb)
        ix = Ix()
        st = lib.pqhsa_index_layout_of(p, ctypes.byref(ix))
        assert (st == OK) == ok_sparse
        if st == OK:
            check_offsets([ix.centroids, ix.codebooks, ix.list_off, ix.codes, ix.pos, ix.means,
                           ix.n_indexed, ix.dropped], lib.pqhsa_index_bytes(p), "index")
        for w in (0, 1, 7, 1024, 8192, 8193, -3):
            ru = Ru()
            st = lib.pqhsa_reuse_layout_of(p, w, ctypes.byref(ru))
            rb = lib.pqhsa_reuse_buffer_bytes(p, w)
            rw = lib.pqhsa_reuse_workspace_bytes(p, w)
            if st == OK:
                assert rb == ru.total > 0 and rw > 0
                check_offsets([ru.search, ru.states, ru.context, ru.count], ru.total, "reuse")
            else:
                assert rb == 0 and rw == 0
        return ok_sparse

    # valid shapes: every group size, short to very long contexts
    for G in (1, 2, 4, 8):
        for T in (1, 16, 4095, 131072, 1 << 20):
            s = shape(num_q_heads=8 * G, num_kv_heads=8, max_context=T,
                      num_pages=(T + 15) // 16, max_pages_per_seq=(T + 15) // 16)
            assert exercise(s), (G, T)
    # invalid or unsupported shapes and arguments
    bad = [dict(batch=0), dict(num_q_heads=-1), dict(num_kv_heads=0), dict(num_q_heads=24),
           dict(num_q_heads=48, num_kv_heads=8), dict(head_dim=64), dict(page_size=32),
           dict(num_pages=0), dict(max_pages_per_seq=0), dict(max_context=0),
           dict(max_context=8193), dict(scale=0.0), dict(scale=-1.0), dict(scale=float("nan")),
           dict(scale=float("inf")), dict(num_lists=0), dict(num_lists=16385), dict(pq_m=8),
           dict(pq_ksub=16), dict(n_sink=-1), dict(n_recent=-5), dict(budget_bp=-1),
           dict(budget_bp=10001), dict(exact_only=2),
           dict(max_context=(1 << 26) + 16, num_pages=1 << 22, max_pages_per_seq=(1 << 22) + 1),
           dict(num_pages=(1 << 27) + 1), dict(num_q_heads=2 ** 31 - 1, num_kv_heads=1),
           dict(max_context=(1 << 20) + 16, max_pages_per_seq=(1 << 16) + 1)]
    for kw in bad:
        s = shape(**kw)
        assert not exercise(s), kw
        assert lib.pqhsa_index_bytes(ctypes.byref(s)) == 0, kw
    # null shape and null outputs
    assert lib.pqhsa_index_bytes(None) == 0 and lib.pqhsa_workspace_bytes(None, 0) == 0
    assert lib.pqhsa_max_selected(None) == 0
    assert lib.pqhsa_workspace_layout(None, 0, None) == INVALID
    s = shape()
    assert lib.pqhsa_workspace_layout(ctypes.byref(s), 0, None) == INVALID
    assert lib.pqhsa_index_layout_of(ctypes.byref(s), None) == INVALID
    assert lib.pqhsa_reuse_layout_of(ctypes.byref(s), 16, None) == INVALID
    # every status has a message, unknown ones too
    for st in (0, 1, 2, 3, 4, 99, -1):
        assert lib.pqhsa_status_string(st)
    # random shapes, fields drawn from small, boundary and extreme values
    rng = random.Random(1234)
    pick = [0, 1, 2, 3, 4, 7, 8, 16, 64, 128, 255, 256, 4096, 65535, 1 << 20, (1 << 26) + 1,
            2 ** 31 - 1, -1, -(2 ** 31)]
    n_valid = 0
    for _ in range(3000):
        kw = {f: rng.choice(pick) for f in SHAPE_FIELDS[:-2]}
        if rng.random() < 0.5:
            kw.update(head_dim=128, page_size=16, pq_m=16, pq_ksub=256)
            kw["num_kv_heads"] = rng.choice([1, 2, 8, 64])
            kw["num_q_heads"] = kw["num_kv_heads"] * rng.choice([1, 2, 4, 8])
            kw["max_context"] = rng.choice([1, 100, 8192, 131072])
            kw["max_pages_per_seq"] = (kw["max_context"] + 15) // 16 + rng.choice([0, 3])
            kw["num_pages"] = kw["max_pages_per_seq"] * rng.choice([1, 4])
            kw["batch"] = rng.choice([1, 3, 16])
            kw["num_lists"] = rng.choice([1, 64, 2048, 16384])
            kw["budget_bp"] = rng.choice([0, 100, 10000])
            kw["n_sink"], kw["n_recent"] = rng.choice([0, 4]), rng.choice([0, 256])
        kw["scale"] = rng.choice([0.088, 1.0, 0.0, float("nan"), 1e-30])
        kw["exact_only"] = rng.choice([0, 1, 3])
        n_valid += exercise(Shape(**kw))
    assert n_valid > 100, n_valid
    print("host sanitizer driver ok:", n_valid, "valid random shapes")
''')


def _sanitizer_runtime():
    gxx = shutil.which("g++")
    if not gxx:
        return None, None
    asan = subprocess.run([gxx, "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    if not asan or not os.path.isabs(asan) or not os.path.exists(asan):
        return gxx, None
    return gxx, asan


def test_driver_structs_match_the_package():
    lib = pytest.importorskip("ivf_pq_sparse_amd._lib")
    assert [n for n, _ in lib.Shape._fields_] == SHAPE_FIELDS
    assert [n for n, _ in lib.WsLayout._fields_] == WS_FIELDS
    assert [n for n, _ in lib.IndexLayout._fields_] == INDEX_FIELDS
    assert [n for n, _ in lib.ReuseLayout._fields_] == REUSE_FIELDS


def test_host_logic_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    gxx, asan = _sanitizer_runtime()
    if gxx is None or asan is None:
        pytest.skip("g++ with the AddressSanitizer runtime is not available")
    so = tmp_path / "libpqhsa_host_san.so"
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-Wall", "-Wextra", "-Werror",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-shared", "-fPIC", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
           os.path.join(CSRC, "pqhsa_host.cpp"), "-o", str(so)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    drv = tmp_path / "driver.py"
    drv.write_text(f"SHAPE_FIELDS = {SHAPE_FIELDS!r}\nWS_FIELDS = {WS_FIELDS!r}\n"
                   f"INDEX_FIELDS = {INDEX_FIELDS!r}\nREUSE_FIELDS = {REUSE_FIELDS!r}\n" + DRIVER)
    env = dict(os.environ, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, str(drv), str(so)], capture_output=True, text=True,
                       env=env, timeout=600)
    report = r.stdout[-2000:] + r.stderr[-6000:]
    assert r.returncode == 0, report
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, report
    assert "host sanitizer driver ok" in r.stdout, report
