"""Write tests/golden/pool_enum.json: a digest of what the oracle's pool model (oracle.pool.
PoolModel) does on every sequence of at most DEPTH operations from a fixed alphabet, on a
4-block pool whose tables hold 3 blocks ("KV Cache and PagedAttention", sections 2.1, 3.1, 3.3
and 5.1: first fit, reference counts, fork and copy-on-write; "KV Cache Mechanism Explained",
section 8 item 2: the rolling window's slide).

The sequences are visited depth first, children in alphabet order. After each operation the
outcome (status, the call's results, the statistics, every live sequence's length and table) is
folded into a 64-bit FNV-1a hash over 64-bit words. tests/pool_enum.cpp visits the same tree
with the library's C pool and must reach the same hash and node count.

Run from the repository root: python tests/golden/make_pool_enum.py  (about two minutes).
Only oracle/ is used.
"""
from __future__ import annotations

import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle.pool import PoolError, PoolModel  # noqa: E402

NUM_BLOCKS, MAX_BLOCKS, DEPTH = 4, 3, int(os.environ.get("POOL_ENUM_DEPTH", "6"))

# (kind, argument): sequence arguments are indices into the list of live sequences (mod its
# length); with no live sequence, append/slide name sequence 0 and fork/free sequence 7
ALPHABET = ([("alloc", None)] + [("append", ([0], n)) for n in (1, 15, 17)]
            + [("append", ([0, 1], 1)), ("append", ([1, 0], 9))]
            + [("fork", 0), ("fork", 1), ("free", 0), ("free", 1)]
            + [("slide", ([0], 3)), ("slide", ([1, 0], 17))])

MASK = (1 << 64) - 1
FNV_OFFSET, FNV_PRIME = 0xCBF29CE484222325, 0x100000001B3


def fold(h: int, words) -> int:
    for v in words:
        h = ((h ^ (int(v) & MASK)) * FNV_PRIME) & MASK
    return h


def snapshot(m: PoolModel, live):
    return (list(m.refcount), {s: {"len": q["len"], "table": list(q["table"])}
                               for s, q in m.seqs.items()}, m.cow_copies, list(live))


def restore(m: PoolModel, snap):
    m.refcount = list(snap[0])
    m.seqs = {s: {"len": q["len"], "table": list(q["table"])} for s, q in snap[1].items()}
    m.cow_copies = snap[2]
    return list(snap[3])


def apply(m: PoolModel, live, op):
    """Apply one operation; returns (status, result words, new live list)."""
    kind, arg = op
    try:
        if kind == "alloc":
            s = m.alloc()
            return 0, [s], live + [s]
        if kind == "append":
            idx, n = arg
            seqs = [live[i % len(live)] for i in idx] if live else [0]
            slots, cow = m.append(seqs, n)
            return 0, [len(slots)] + slots + [len(cow)] + [x for p in cow for x in p], live
        if kind == "fork":
            s = live[arg % len(live)] if live else 7
            c = m.fork(s)
            return 0, [c], live + [c]
        if kind == "free":
            s = live[arg % len(live)] if live else 7
            m.free(s)
            return 0, [], [x for x in live if x != s]
        idx, w = arg
        seqs = [live[i % len(live)] for i in idx] if live else [0]
        return 0, [m.slide(seqs, w)], live
    except PoolError as e:
        return e.code, [], live


def outcome(m: PoolModel, live, depth, op_i, status, res):
    st = m.stats()
    words = [depth, op_i, status] + res
    words += [st["num_blocks"], st["used"], st["free"], st["shared"], st["num_seqs"],
              st["cow_copies"], st["tokens"], st["slots_logical"], len(live)]
    if live:
        tables, lens = m.block_table(live)
        for t, L in zip(tables, lens):
            words += [L] + t
    return words


def main():
    m = PoolModel(NUM_BLOCKS, 16, MAX_BLOCKS)
    h = FNV_OFFSET
    nodes = [0] * (DEPTH + 1)
    errors = 0

    def visit(live, depth):
        nonlocal h, errors
        snap = snapshot(m, live)
        for op_i, op in enumerate(ALPHABET):
            cur = restore(m, snap)
            status, res, cur = apply(m, cur, op)
            m.check()
            h = fold(h, outcome(m, cur, depth, op_i, status, res))
            nodes[depth] += 1
            errors += status != 0
            if depth < DEPTH:
                visit(cur, depth + 1)
        restore(m, snap)

    visit([], 1)
    rec = {"num_blocks": NUM_BLOCKS, "max_blocks_per_seq": MAX_BLOCKS, "depth": DEPTH,
           "alphabet_size": len(ALPHABET), "nodes_per_depth": nodes[1:],
           "failed_calls": errors, "fnv1a64": f"{h:016x}"}
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "pool_enum.json")
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
