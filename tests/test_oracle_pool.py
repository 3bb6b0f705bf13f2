"""Pins for oracle.pool.PoolModel (CPU only): the pages' printed block counts, a hand-traced
copy-on-write scenario, the growth trace, error cases, and invariants under random operations."""
import json
import os

import numpy as np
import pytest

from oracle.pool import (E_CAPACITY, E_INVALID, E_NOSEQ, E_OOM, PoolError, PoolModel)

FIG = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))


def test_growth_trace_prompt_then_two_steps():
    g = FIG["growth_trace"]
    p = PoolModel(8, 16, 4)
    s = p.alloc()
    slots, cow = p.append([s], g["prompt_tokens"])
    assert slots == [0, 1, 2] and cow == []
    lens = [p.block_table([s])[1][0]]
    for _ in range(2):
        slots, _ = p.append([s], 1)
        lens.append(p.block_table([s])[1][0])
    assert lens == g["cache_lengths"]
    assert slots == [4]


def test_block_count_and_waste_at_1024_tokens():
    f = FIG["block16_t1024"]
    p = PoolModel(128, 16, 128)
    s = p.alloc()
    p.append([s], 1024)
    st = p.stats()
    assert st["used"] == f["blocks"]
    # the worst case over lengths is one token into a fresh block
    worst = 0
    for T in range(1, 1100):
        q = PoolModel(80, 16, 80)
        t = q.alloc()
        q.append([t], T)
        worst = max(worst, q.stats()["slots_logical"] - T)
    assert worst == f["max_waste_tokens"]
    assert abs(worst / 1024 - f["waste_fraction_approx"]) < 0.001


def _sampling(prompt, gen, n=8, shared=True):
    p = PoolModel(1024, 16, 128)
    parent = p.alloc()
    p.append([parent], prompt)
    seqs = [parent]
    if shared:
        seqs += [p.fork(parent) for _ in range(n - 1)]
    else:
        for _ in range(n - 1):
            s = p.alloc()
            p.append([s], prompt)
            seqs.append(s)
    copies = []
    for _ in range(gen):
        _, cow = p.append(seqs, 1)
        copies.append(len(cow))
        p.check()
    return p, seqs, copies


def test_parallel_sampling_capacity_matches_page():
    f = FIG["parallel_sampling"]
    p, seqs, copies = _sampling(f["prompt"], f["generated"], f["candidates"], shared=True)
    st = p.stats()
    assert st["used"] * 16 == f["capacity_shared"]
    assert st["tokens"] == f["candidates"] * (f["prompt"] + f["generated"])
    assert sum(copies) == 0           # 1024 is a whole number of blocks: nothing partial is shared
    u, _, _ = _sampling(f["prompt"], f["generated"], f["candidates"], shared=False)
    assert u.stats()["used"] * 16 == f["capacity_unshared"]
    saving = (f["capacity_unshared"] - f["capacity_shared"]) / f["capacity_unshared"]
    assert abs(saving - f["saving_approx"]) < 0.005


def test_parallel_sampling_partial_prompt_block_copy_on_write():
    p, seqs, copies = _sampling(1020, 128, 8, shared=True)
    # first step: candidates 0..6 copy the shared partial block; the last holder writes in place
    assert copies[0] == 7 and sum(copies) == 7
    st = p.stats()
    assert st["used"] == 63 + 8 * 9 == 135
    assert st["cow_copies"] == 7
    tables, lens = p.block_table(seqs)
    assert all(L == 1148 for L in lens)
    assert len({tuple(t[:63]) for t in tables}) == 1        # full prompt blocks still shared
    assert len({t[63] for t in tables}) == 8                 # the partial block is now private


def test_hand_traced_copy_on_write():
    p = PoolModel(6, 16, 4)
    a = p.alloc()
    assert p.append([a], 20)[0] == list(range(16)) + [16, 17, 18, 19]   # blocks 0, 1
    b = p.fork(a)
    assert b == 1 and p.refcount[:3] == [2, 2, 0]
    # b writes first: its partial block 1 is shared -> copy into block 2
    slots, cow = p.append([b, a], 1)
    assert cow == [(1, 2)]
    assert slots == [2 * 16 + 4, 1 * 16 + 4]        # a is now the only holder of block 1
    t, lens = p.block_table([a, b])
    assert t == [[0, 1, -1, -1], [0, 2, -1, -1]] and lens == [21, 21]
    assert p.refcount == [2, 1, 1, 0, 0, 0]
    p.free(a)
    assert p.refcount == [1, 0, 1, 0, 0, 0]
    c = p.alloc()
    assert c == 0                       # lowest free sequence id is reused
    assert p.append([c], 1)[0] == [16]  # first fit: block 1 is the first free block
    p.check()


def test_first_fit_follows_pool_order():
    order = [5, 2, 7, 0, 1, 3, 4, 6]
    p = PoolModel(8, 16, 8, order=order)
    s = p.alloc()
    p.append([s], 16 * 3)
    assert p.block_table([s])[0][0][:3] == [5, 2, 7]
    t = p.alloc()
    p.append([t], 1)
    assert p.block_table([t])[0][0][0] == 0
    p.free(s)
    u = p.alloc()
    p.append([u], 1)
    assert p.block_table([u])[0][0][0] == 5


def test_errors_leave_state_unchanged():
    p = PoolModel(4, 16, 2)
    a, b = p.alloc(), p.alloc()
    p.append([a], 16)
    before = (list(p.refcount), {k: dict(v, table=list(v["table"])) for k, v in p.seqs.items()})
    with pytest.raises(PoolError) as e:
        p.append([a], 17)            # a would need a third block: table capacity 2
    assert e.value.code == E_CAPACITY
    with pytest.raises(PoolError) as e:
        p.append([b, a], 40)         # b takes 3 blocks: only 3 free, then a needs more
    assert e.value.code in (E_OOM, E_CAPACITY)
    with pytest.raises(PoolError) as e:
        p.append([a, 9], 1)
    assert e.value.code == E_NOSEQ
    after = (list(p.refcount), {k: dict(v, table=list(v["table"])) for k, v in p.seqs.items()})
    assert before == after
    with pytest.raises(PoolError) as e:
        p.fork(7)
    assert e.value.code == E_NOSEQ
    p.free(b)
    with pytest.raises(PoolError) as e:
        p.free(b)
    assert e.value.code == E_NOSEQ
    with pytest.raises(PoolError) as e:
        PoolModel(4, 8, 2)
    assert e.value.code == E_INVALID
    q = PoolModel(2, 16, 8)
    s = q.alloc()
    with pytest.raises(PoolError) as e:
        q.append([s], 33)
    assert e.value.code == E_OOM
    assert q.stats()["used"] == 0


def test_random_operations_keep_invariants():
    rng = np.random.default_rng(5)
    for trial in range(30):
        p = PoolModel(int(rng.integers(1, 12)), 16, int(rng.integers(1, 5)))
        live = []
        for _ in range(60):
            op = rng.integers(0, 4)
            try:
                if op == 0 or not live:
                    live.append(p.alloc())
                elif op == 1:
                    k = int(rng.integers(1, len(live) + 1))
                    p.append(list(rng.choice(live, k, replace=False)), int(rng.integers(0, 20)))
                elif op == 2:
                    live.append(p.fork(int(rng.choice(live))))
                else:
                    s = int(rng.choice(live))
                    p.free(s)
                    live.remove(s)
            except PoolError as e:
                assert e.code in (E_OOM, E_CAPACITY)
            p.check()
            st = p.stats()
            assert st["used"] + st["free"] == p.num_blocks
