"""PoolModel: the paged KV cache's block bookkeeping, in plain Python.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

What it models ("KV Cache and PagedAttention", sections 2.1, 3.1 and 3.3; "LLM Inference
Acceleration -- KV Cache", section 6.1):
  * one global pool of fixed-size physical blocks (16 tokens each, section 2.2);
  * one block table per sequence mapping logical block i (tokens 16i .. 16i+15) to a physical
    block id; one table per sequence serves every layer;
  * a reference count per physical block; refcount > 1 means the block is shared;
  * allocation by first fit: the first free block in pool order (section 3.1 picks first fit
    over best fit). Pool order is block id order unless a permutation is given, which models a
    shuffled pool. Blocks are all one size, so no buddy coalescing applies;
  * fork: a new sequence sharing all of a parent's blocks (parallel sampling, section 5.1);
  * copy-on-write (section 3.3): writing into a block whose refcount > 1 first takes a fresh
    block, records a (src, dst) copy, drops one reference to src and repoints the table;
  * free: drop one reference per block; a block whose count reaches 0 is free again (its
    contents are left as they are);
  * slide: the rolling window of "KV Cache Mechanism Explained", section 8, item 2, in paged
    form: a block all of whose positions lie before the window is dropped from the sequence
    (one reference released, its table entry set to -1). Positions stay absolute: the length
    keeps counting every token appended, and dropped entries form a prefix of the table.

Readings where the pages are silent: sequence ids are the lowest id not in use; appends for
several sequences are applied in the order given, all tokens of one sequence before the next;
a failed call (out of blocks, table full, unknown sequence) changes nothing.
"""
from __future__ import annotations

import copy

OK = 0
E_INVALID = -1
E_OOM = -2
E_NOSEQ = -3
E_CAPACITY = -4


class PoolError(Exception):
    def __init__(self, code: int, msg: str = ""):
        super().__init__(f"{code}: {msg}")
        self.code = code


class PoolModel:
    def __init__(self, num_blocks: int, block_size: int = 16, max_blocks_per_seq: int = 1,
                 order=None):
        if num_blocks < 1 or block_size != 16 or max_blocks_per_seq < 1:
            raise PoolError(E_INVALID, "bad pool shape")
        if order is None:
            order = list(range(num_blocks))
        order = [int(b) for b in order]
        if sorted(order) != list(range(num_blocks)):
            raise PoolError(E_INVALID, "order is not a permutation")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.max_blocks_per_seq = max_blocks_per_seq
        self.order = order
        self.refcount = [0] * num_blocks
        self.seqs: dict[int, dict] = {}
        self.cow_copies = 0

    # -- helpers ------------------------------------------------------------------------------
    def _first_fit(self):
        for b in self.order:
            if self.refcount[b] == 0:
                return b
        return None

    def _state(self):
        return copy.deepcopy((self.refcount, self.seqs, self.cow_copies))

    def _restore(self, st):
        self.refcount, self.seqs, self.cow_copies = st

    def _need(self, s: int):
        if s not in self.seqs:
            raise PoolError(E_NOSEQ, f"sequence {s} is not live")
        return self.seqs[s]

    # -- operations ---------------------------------------------------------------------------
    def alloc(self) -> int:
        sid = 0
        while sid in self.seqs:
            sid += 1
        self.seqs[sid] = {"len": 0, "table": []}
        return sid

    def append(self, seqs, n_tokens: int):
        """Reserve n_tokens new slots at the end of each sequence. Returns (slots, cow_pairs):
        slots[i*n_tokens + j] = physical_block*16 + in-block offset of token j of seqs[i]."""
        if n_tokens < 0:
            raise PoolError(E_INVALID, "negative token count")
        for s in seqs:
            self._need(s)
        saved = self._state()
        slots, cow = [], []
        bs = self.block_size
        try:
            for s in seqs:
                seq = self.seqs[s]
                for _ in range(n_tokens):
                    L = seq["len"]
                    idx, off = divmod(L, bs)
                    if off == 0:
                        if idx >= self.max_blocks_per_seq:
                            raise PoolError(E_CAPACITY, "block table full")
                        b = self._first_fit()
                        if b is None:
                            raise PoolError(E_OOM, "no free block")
                        self.refcount[b] = 1
                        seq["table"].append(b)
                    else:
                        b = seq["table"][idx]
                        if self.refcount[b] > 1:
                            nb = self._first_fit()
                            if nb is None:
                                raise PoolError(E_OOM, "no free block for copy-on-write")
                            self.refcount[nb] = 1
                            self.refcount[b] -= 1
                            seq["table"][idx] = nb
                            cow.append((b, nb))
                            self.cow_copies += 1
                            b = nb
                    slots.append(b * bs + off)
                    seq["len"] = L + 1
        except PoolError:
            self._restore(saved)
            raise
        return slots, cow

    def fork(self, parent: int) -> int:
        p = self._need(parent)
        child = self.alloc()
        self.seqs[child] = {"len": p["len"], "table": list(p["table"])}
        for b in p["table"]:
            if b >= 0:
                self.refcount[b] += 1
        return child

    def free(self, s: int) -> None:
        seq = self._need(s)
        for b in seq["table"]:
            if b >= 0:
                self.refcount[b] -= 1
        del self.seqs[s]

    def slide(self, seqs, window: int) -> int:
        """Rolling window: for each listed sequence, drop every block whose 16 positions all lie
        before the window's first position max(0, len - window), i.e. logical blocks
        0 .. (len - window) // 16 - 1 still held. Each dropped entry releases one reference and
        becomes -1. window 0 drops nothing. Returns the number of entries dropped."""
        if window < 0:
            raise PoolError(E_INVALID, "negative window")
        for s in seqs:
            self._need(s)
        dropped = 0
        if window == 0:
            return 0
        for s in seqs:
            seq = self.seqs[s]
            start = max(0, seq["len"] - window)
            for i in range(start // self.block_size):
                b = seq["table"][i]
                if b >= 0:
                    self.refcount[b] -= 1
                    seq["table"][i] = -1
                    dropped += 1
        return dropped

    def block_table(self, seqs):
        """Per sequence: the table padded with -1 to max_blocks_per_seq, and the length."""
        tables, lens = [], []
        for s in seqs:
            seq = self._need(s)
            t = list(seq["table"]) + [-1] * (self.max_blocks_per_seq - len(seq["table"]))
            tables.append(t)
            lens.append(seq["len"])
        return tables, lens

    def stats(self) -> dict:
        used = sum(1 for r in self.refcount if r > 0)
        return {
            "num_blocks": self.num_blocks,
            "used": used,
            "free": self.num_blocks - used,
            "shared": sum(1 for r in self.refcount if r > 1),
            "num_seqs": len(self.seqs),
            "cow_copies": self.cow_copies,
            "tokens": sum(s["len"] for s in self.seqs.values()),
            "slots_logical": sum(sum(1 for b in s["table"] if b >= 0) * self.block_size
                                 for s in self.seqs.values()),
        }

    def check(self) -> None:
        """Raise PoolError(E_INVALID) unless every invariant holds: each block's refcount equals
        the number of table entries naming it; each table has exactly ceil(len/16) entries,
        within the table capacity, in range and without repeats, except a prefix of entries
        dropped by slide (-1)."""
        refs = [0] * self.num_blocks
        for sid, s in self.seqs.items():
            t = s["table"]
            need = -(-s["len"] // self.block_size)
            if len(t) != need or len(t) > self.max_blocks_per_seq:
                raise PoolError(E_INVALID, f"sequence {sid}: table size")
            k = 0
            while k < len(t) and t[k] == -1:
                k += 1
            t = t[k:]
            if len(set(t)) != len(t):
                raise PoolError(E_INVALID, f"sequence {sid}: repeated block")
            for b in t:
                if not 0 <= b < self.num_blocks:
                    raise PoolError(E_INVALID, f"sequence {sid}: block out of range")
                refs[b] += 1
        if refs != self.refcount:
            raise PoolError(E_INVALID, "refcounts disagree with tables")
