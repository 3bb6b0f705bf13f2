"""libkvc host side on the CPU: the shared library loads and exports every symbol that
include/kvc.h declares, and the C++ block pool matches oracle.pool.PoolModel bit for bit
(tables, lengths, slots, copy-on-write pairs, statistics, error codes). No GPU calls."""
import ctypes
import itertools
import os
import re

import numpy as np
import pytest

import kv_cache_attention_kvc_amd as kvc
from oracle.pool import PoolError, PoolModel

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", autouse=True)
def lib():
    if not os.path.exists(kvc.library_path()):
        from kv_cache_attention_kvc_amd.csrc.build import build
        build()
    return kvc.load_library()


def test_exports_every_declared_symbol(lib):
    hdr = open(os.path.join(ROOT, "include", "kvc.h")).read()
    declared = set(re.findall(r"\b(kvc_[a-z_]+)\s*\(", hdr))
    assert declared == set(kvc.EXPORTS)
    for name in declared:
        assert getattr(lib, name) is not None
    assert lib.kvc_status_str(-4).decode() == "block table full"


def test_merge_needed_query_checks_its_arguments(lib):
    """kvc_decode_merge_needed rejects what the matching pass-1 call rejects, before any runtime
    call: a null result pointer, 8-bit contiguous caches, 8-bit fused appends, a window with the
    fused append, a negative batch; B = 0 needs no merge."""
    f = lib.kvc_decode_merge_needed
    res = ctypes.c_int32(7)
    assert f(1, 0, kvc.F16, kvc.F16, 4, 8, 1, 128, 256, 256, 0, None) == -1
    assert f(0, 0, kvc.F16, kvc.E4M3, 4, 8, 1, 128, 256, 256, 0, ctypes.byref(res)) == -5
    assert f(1, 1, kvc.F16, kvc.I8, 4, 8, 1, 128, 256, 256, 0, ctypes.byref(res)) == -5
    assert f(1, 1, kvc.F16, kvc.F16, 4, 8, 1, 128, 256, 256, 64, ctypes.byref(res)) == -1
    assert f(1, 0, kvc.F16, kvc.F16, -1, 8, 1, 128, 256, 256, 0, ctypes.byref(res)) == -1
    assert f(1, 0, kvc.F16, kvc.F16, 0, 8, 1, 128, 256, 256, 0, ctypes.byref(res)) == 0
    assert res.value == 0
    assert not kvc.decode_merge_needed(True, "f16", "f16", 0, 40, 128, 2064, 2064)


def test_workspace_size_is_monotone(lib):
    a = kvc.workspace_bytes(32, 40, 128)
    assert a > 0 and kvc.workspace_bytes(64, 40, 128) >= a
    assert kvc.workspace_bytes(32, 40, 64) < a


class Mirror:
    """Drive the C++ pool and PoolModel with the same operations and compare everything."""

    def __init__(self, nblk, mbps, order=None):
        self.c = kvc.Pool(nblk, mbps, order=order)
        self.p = PoolModel(nblk, 16, mbps, order=order)
        self.live = []

    def _both(self, fc, fp):
        try:
            rc = ("ok", fc())
        except kvc.KvcError as e:
            rc = ("err", e.status)
        try:
            rp = ("ok", fp())
        except PoolError as e:
            rp = ("err", e.code)
        return rc, rp

    def op(self, kind, arg):
        if kind == "alloc":
            rc, rp = self._both(self.c.alloc, self.p.alloc)
            assert rc == rp
            if rc[0] == "ok":
                self.live.append(rc[1])
        elif kind == "append":
            seqs, n = arg
            seqs = [self.live[i % len(self.live)] for i in seqs] if self.live else [0]
            rc, rp = self._both(lambda: self.c.append(seqs, n), lambda: self.p.append(seqs, n))
            assert rc[0] == rp[0], (rc, rp)
            if rc[0] == "ok":
                slots, src, dst = rc[1]
                assert list(slots) == rp[1][0]
                assert list(zip(src.tolist(), dst.tolist())) == rp[1][1]
            else:
                assert rc[1] == rp[1]
        elif kind == "fork":
            s = self.live[arg % len(self.live)] if self.live else 7
            rc, rp = self._both(lambda: self.c.fork(s), lambda: self.p.fork(s))
            assert rc == rp
            if rc[0] == "ok":
                self.live.append(rc[1])
        elif kind == "free":
            s = self.live[arg % len(self.live)] if self.live else 7
            rc, rp = self._both(lambda: self.c.free(s), lambda: self.p.free(s))
            assert rc == rp
            if rc[0] == "ok":
                self.live.remove(s)
        elif kind == "slide":
            seqs, w = arg
            seqs = [self.live[i % len(self.live)] for i in seqs] if self.live else [0]
            rc, rp = self._both(lambda: self.c.slide(seqs, w), lambda: self.p.slide(seqs, w))
            assert rc == rp
        self.compare()

    def compare(self):
        self.c.check()
        self.p.check()
        sc, sp = self.c.stats(), self.p.stats()
        assert sc["free_blocks"] == sp["free"]
        for k in ("num_blocks", "used", "shared", "num_seqs", "cow_copies", "tokens",
                  "slots_logical"):
            assert sc[k] == sp[k], k
        if self.live:
            tc, lc = self.c.block_table(self.live)
            tp, lp = self.p.block_table(self.live)
            assert tc.tolist() == tp and lc.tolist() == lp


OPS = ([("alloc", None)] + [("append", ([0], n)) for n in (1, 15, 17)]
       + [("append", ([0, 1], 1)), ("append", ([1, 0], 9))]
       + [("fork", 0), ("fork", 1), ("free", 0), ("free", 1)]
       + [("slide", ([0], 3)), ("slide", ([1, 0], 17))])


def test_pool_matches_model_on_every_short_op_sequence():
    for length in range(1, 5):
        for seq in itertools.product(range(len(OPS)), repeat=length):
            m = Mirror(4, 3)
            for i in seq:
                m.op(*OPS[i])


def test_pool_matches_model_on_every_op_sequence_up_to_six():
    """Every sequence of at most 6 operations of the same 12-operation alphabet on a 4-block pool
    (tables of 3): the C++ pool, driven through its C ABI by tests/pool_enum.cpp, folds each
    outcome (status, results, statistics, every live table and length) into a hash that must
    equal the one tests/golden/make_pool_enum.py computed with the oracle's PoolModel."""
    import json
    import shutil
    import subprocess
    import tempfile
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    want = json.load(open(os.path.join(ROOT, "tests", "golden", "pool_enum.json")))
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "pool_enum")
        r = subprocess.run(["g++", "-std=c++17", "-O2", "-I", os.path.join(ROOT, "include"),
                            os.path.join(ROOT, "kv_cache_attention_kvc_amd", "csrc",
                                         "kvc_pool.cpp"),
                            os.path.join(ROOT, "tests", "pool_enum.cpp"), "-o", exe],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        r = subprocess.run([exe, str(want["depth"])], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    words = r.stdout.split()
    nodes = [int(x) for x in words[1:1 + want["depth"]]]
    assert nodes == want["nodes_per_depth"]
    assert int(words[words.index("failed") + 1]) == want["failed_calls"]
    assert words[words.index("fnv1a64") + 1] == want["fnv1a64"]


@pytest.mark.parametrize("seed", range(6))
def test_pool_matches_model_on_random_long_sequences(seed):
    rng = np.random.default_rng(seed)
    nblk = int(rng.integers(3, 40))
    order = rng.permutation(nblk) if seed % 2 else None
    m = Mirror(nblk, int(rng.integers(1, 6)), order=order)
    for _ in range(150):
        k = rng.integers(0, 11)
        if k < 2:
            m.op("alloc", None)
        elif k < 6:
            nseq = int(rng.integers(1, 4))
            m.op("append", (list(rng.integers(0, 8, nseq)), int(rng.integers(0, 24))))
        elif k < 8:
            m.op("fork", int(rng.integers(0, 8)))
        elif k < 9:
            m.op("free", int(rng.integers(0, 8)))
        else:
            nseq = int(rng.integers(1, 4))
            m.op("slide", (list(rng.integers(0, 8, nseq)), int(rng.integers(0, 40))))


def test_pool_argument_errors(lib):
    h = ctypes.c_void_p()
    assert lib.kvc_pool_create(0, 16, 4, None, ctypes.byref(h)) == -1
    assert lib.kvc_pool_create(4, 8, 4, None, ctypes.byref(h)) == -1
    bad = np.array([0, 0, 1, 2], dtype=np.int32)
    assert lib.kvc_pool_create(4, 16, 4, bad.ctypes.data, ctypes.byref(h)) == -1
    p = kvc.Pool(4, 2)
    s = p.alloc()
    slots = np.empty(4, dtype=np.int64)
    src = np.empty(1, dtype=np.int32)
    n = ctypes.c_int32()
    seqs = np.array([s, s], dtype=np.int32)
    # cow_cap below the number of listed sequences is refused
    assert lib.kvc_append(p._h, seqs.ctypes.data, 2, 1, slots.ctypes.data, src.ctypes.data,
                          src.ctypes.data, 1, ctypes.byref(n)) == -1
    assert lib.kvc_check(p._h) == 0


def test_parallel_sampling_counts_through_library():
    p = kvc.Pool(1024, 128)
    parent = p.alloc()
    p.append([parent], 1020)
    seqs = [parent] + [p.fork(parent) for _ in range(7)]
    _, src, dst = p.append(seqs, 1)
    assert len(src) == 7 and len(set(dst.tolist())) == 7
    for _ in range(127):
        p.append(seqs, 1)
    st = p.stats()
    assert st["used"] == 135 and st["cow_copies"] == 7


def test_binding_refuses_index_tensors_of_the_wrong_width():
    """Block tables, lengths, positions and block ids are int32 and slots int64 in the C ABI; a
    tensor of another integer width is refused before any call (its bytes would otherwise be
    read as a different layout)."""
    import torch
    for name, good, bad in (("_ptr_i32", torch.int32, torch.int64), ("_ptr_i64", torch.int64,
                                                                     torch.int32)):
        fn = getattr(kvc, name)
        width = "int32" if good == torch.int32 else "int64"
        # the right width passes the dtype check (and then needs device memory)
        with pytest.raises(ValueError, match="device memory"):
            fn(torch.zeros(4, dtype=good))
        for wrong in (bad, torch.float32):
            with pytest.raises(ValueError, match=f"must be {width}"):
                fn(torch.zeros(4, dtype=wrong))


def test_binding_checks_shapes_before_any_call():
    """The C ABI cannot see the size of a device array, so the binding checks every shape it
    can before a call: q against the cache, one length per sequence, q_start of B + 1 entries,
    and a caller's out of q's shape (or the merge's row count). CPU tensors suffice: each check
    raises before any pointer is taken."""
    import torch
    B, H, D, S = 3, 4, 64, 32
    q = torch.zeros((B, H, D), dtype=torch.float16)
    kc = torch.zeros((B, H, S, D), dtype=torch.float16)
    lens = torch.zeros(B, dtype=torch.int32)
    layer = kvc.PagedLayer(torch.zeros((8, H, 16, D), dtype=torch.float16),
                           torch.zeros((8, H, 16, D), dtype=torch.float16))
    tables = torch.zeros((B, 2), dtype=torch.int32)
    for fn in (kvc.decode_attn_contig, kvc.decode_partial_contig):
        with pytest.raises(ValueError, match="q must be"):
            fn(q[:, :2].contiguous(), kc, kc, lens, S)
        with pytest.raises(ValueError, match="ctx_lens must be"):
            fn(q, kc, kc, lens[:2], S)
        with pytest.raises(ValueError, match="out must have"):
            fn(q, kc, kc, lens, S, out=torch.zeros((B, H, D - 1)))
        with pytest.raises(ValueError, match="out must be float32 or float16"):
            fn(q, kc, kc, lens, S, out=torch.zeros((B, H, D), dtype=torch.int32))
    for fn in (kvc.decode_attn_paged, kvc.decode_partial_paged):
        with pytest.raises(ValueError, match="q must be"):
            fn(torch.zeros((B, H, 2 * D), dtype=torch.float16), layer, tables, lens, S)
        with pytest.raises(ValueError, match="block_tables must be"):
            fn(q, layer, tables[:1], lens, S)
        with pytest.raises(ValueError, match="ctx_lens must be"):
            fn(q, layer, tables, torch.zeros(B + 1, dtype=torch.int32), S)
        with pytest.raises(ValueError, match="out must have"):
            fn(q, layer, tables, lens, S, out=torch.zeros((B + 1, H, D)))
    kn = torch.zeros((B, H, D), dtype=torch.float16)
    with pytest.raises(ValueError, match="ctx_lens must be"):
        kvc.append_decode_partial_paged(q, layer, tables, lens[:1], kn, kn, S)
    with pytest.raises(ValueError, match="q must be"):
        kvc.append_decode_contig(q[:2].contiguous(), kc, kc, lens, kn, kn, S)
    with pytest.raises(ValueError, match="ctx_lens must be"):
        kvc.decode_gqa_paged(torch.zeros((B, 2 * H, D), dtype=torch.float16), layer, tables,
                             lens[:2], S)
    with pytest.raises(ValueError, match="out must have"):
        kvc.decode_window_contig(q, kc, kc, lens, S, 8, out=torch.zeros((B, 2 * H, D)))
    with pytest.raises(ValueError, match="q_start must be"):
        kvc.prefill_paged(q, layer, tables, torch.zeros(B, dtype=torch.int32), lens)
    with pytest.raises(ValueError, match="q_start must be"):
        kvc.prefill_contig(q, kc, kc, torch.zeros(B + 2, dtype=torch.int32), lens)
    with pytest.raises(ValueError, match="out must hold"):
        kvc.decode_merge(B, H, D, torch.zeros((B, H - 1, D)), torch.zeros(16, dtype=torch.uint8))
    with pytest.raises(ValueError, match="out must hold"):
        kvc.decode_gqa_merge(B, H, 2, D, q, torch.zeros(16, dtype=torch.uint8))
