"""Cache storage models and decode through them (fp64 arithmetic).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

ContigCache: one [B, H, S_max, D] array for K and one for V per layer, preallocated to the
maximum length ("LLM Inference Acceleration -- KV Cache", section 3.1, cache_k/cache_v sized
max_batch x max_seq; "KV Cache Mechanism Explained", section 6.2, item 2 -- preallocate the
cache). The new token of sequence b is written at position len_b, then the query attends
positions [0, len_b] (section 3.1: write at start_pos, read up to start_pos + seqlen).

PagedCache: K and V pools [num_blocks, H, 16, D] per layer; token t of a sequence lives in
physical block table[t // 16] at in-block slot t % 16 ("KV Cache and PagedAttention", section
2.1 and section 3.2: gather the sequence's blocks through its block table). Writes go to slots
(physical_block * 16 + offset). Copy-on-write copies whole blocks (section 3.3). An fp8 (int8) pool
keeps uint8 e4m3 (int8) codes plus one fp32 scale per block for K and one for V (codecs module).
"""
from __future__ import annotations

import numpy as np

from .attention import decode_row, full_causal, grouped_decode, kv_head_of, window_start
from .codecs import compress_block, e4m3_decode, fp8_write_token, i8_decode, i8_write_token

BS = 16
_NP = {"f32": np.float32, "f16": np.float16}


class ContigCache:
    def __init__(self, B: int, H: int, S_max: int, D: int, dtype: str, fill=0.0):
        self.B, self.H, self.S_max, self.D = B, H, S_max, D
        self.K = np.full((B, H, S_max, D), fill, dtype=_NP[dtype])
        self.V = np.full((B, H, S_max, D), fill, dtype=_NP[dtype])

    def append(self, pos, k_new, v_new) -> None:
        """k_new, v_new: [B, n, H, D]; token t of sequence b goes to position pos[b] + t.
        Positions outside [0, S_max) are skipped."""
        n = k_new.shape[1]
        for b in range(self.B):
            for t in range(n):
                p = int(pos[b]) + t
                if 0 <= p < self.S_max:
                    self.K[b, :, p, :] = k_new[b, t]
                    self.V[b, :, p, :] = v_new[b, t]

    def decode(self, q, lens, scale, window: int = 0) -> np.ndarray:
        """q: [B, Hq, D] with Hq a multiple of the cache's H (query heads sharing key/value heads
        as in grouped_decode; Hq = H is plain multi-head attention); lens[b]: attended length
        (the new token included); window > 0: only positions window_start(lens[b], window) ..
        lens[b]-1 are attended. Returns [B, Hq, D]."""
        Hq = q.shape[1]
        out = np.zeros((self.B, Hq, self.D))
        for b in range(self.B):
            L = int(lens[b])
            s = window_start(L, window)
            out[b] = grouped_decode(q[b], self.K[b, :, s:L], self.V[b, :, s:L], scale)
        return out

    def prefill(self, q, q_start, lens, scale) -> np.ndarray:
        """Attention of a chunk of new tokens per sequence, their K/V already in the cache.

        q: [total, Hq, D]; sequence b's chunk is rows q_start[b] .. q_start[b+1]-1, the last
        n_b = q_start[b+1] - q_start[b] of its lens[b] positions. Row i attends positions
        0 .. lens[b] - n_b + i (the causal mask of full_causal with start_pos lens[b] - n_b).
        Query head hq reads key/value head kv_head_of(hq, Hq, H). Returns [total, Hq, D]."""
        return _prefill(q, q_start, lens, scale, self.H,
                        lambda b, L: (self.K[b, :, :L], self.V[b, :, :L]))


class PagedCache:
    def __init__(self, num_blocks: int, H: int, D: int, dtype: str, fill=0.0):
        self.N, self.H, self.D, self.dtype = num_blocks, H, D, dtype
        if dtype == "e4m3":
            code = 0x7F if (fill is not None and np.isnan(fill)) else 0   # NaN code poisons
            self.K = np.full((num_blocks, H, BS, D), code, dtype=np.uint8)
            self.V = np.full((num_blocks, H, BS, D), code, dtype=np.uint8)
            self.k_scale = np.zeros(num_blocks, dtype=np.float32)
            self.v_scale = np.zeros(num_blocks, dtype=np.float32)
        elif dtype == "i8":
            # int8 has no NaN; the never-written code -128 marks unused slots
            code = -128 if (fill is not None and np.isnan(fill)) else 0
            self.K = np.full((num_blocks, H, BS, D), code, dtype=np.int8)
            self.V = np.full((num_blocks, H, BS, D), code, dtype=np.int8)
            self.k_scale = np.zeros(num_blocks, dtype=np.float32)
            self.v_scale = np.zeros(num_blocks, dtype=np.float32)
        else:
            self.K = np.full((num_blocks, H, BS, D), fill, dtype=_NP[dtype])
            self.V = np.full((num_blocks, H, BS, D), fill, dtype=_NP[dtype])
            self.k_scale = self.v_scale = None

    def copy_blocks(self, pairs) -> None:
        """Copy every (src, dst) block: all 16 slots of K and V, and the fp8 scales."""
        for s, d in pairs:
            self.K[d] = self.K[s]
            self.V[d] = self.V[s]
            if self.k_scale is not None:
                self.k_scale[d] = self.k_scale[s]
                self.v_scale[d] = self.v_scale[s]

    def compress_from(self, src: "PagedCache", pairs) -> None:
        """One-shot 8-bit compression (codecs.compress_block) of blocks of a 16-bit or fp32 cache
        into this 8-bit cache: pairs of (source block, destination block, valid slots)."""
        if self.dtype not in ("e4m3", "i8") or src.dtype not in ("f16", "f32"):
            raise ValueError("compression goes from a 16/32-bit cache into an 8-bit cache")
        for s, d, n in pairs:
            self.K[d], self.k_scale[d] = compress_block(src.K[s].astype(np.float32), n, self.dtype)
            self.V[d], self.v_scale[d] = compress_block(src.V[s].astype(np.float32), n, self.dtype)

    def write(self, slots, k_new, v_new) -> None:
        """k_new, v_new: [n, H, D]; entry i goes to slot slots[i]; entries are applied in order."""
        for i, slot in enumerate(slots):
            blk, off = divmod(int(slot), BS)
            if self.dtype == "e4m3":
                self.k_scale[blk] = fp8_write_token(self.K[blk], self.k_scale[blk], off, k_new[i])
                self.v_scale[blk] = fp8_write_token(self.V[blk], self.v_scale[blk], off, v_new[i])
            elif self.dtype == "i8":
                self.k_scale[blk] = i8_write_token(self.K[blk], self.k_scale[blk], off, k_new[i])
                self.v_scale[blk] = i8_write_token(self.V[blk], self.v_scale[blk], off, v_new[i])
            else:
                self.K[blk, :, off, :] = k_new[i]
                self.V[blk, :, off, :] = v_new[i]

    def values(self, pool: str, blk: int) -> np.ndarray:
        """Stored values of one block, [H, 16, D] fp64."""
        if self.dtype in ("e4m3", "i8"):
            codes = self.K[blk] if pool == "k" else self.V[blk]
            s = self.k_scale[blk] if pool == "k" else self.v_scale[blk]
            dec = e4m3_decode if self.dtype == "e4m3" else i8_decode
            return dec(codes) * np.float64(s)
        return (self.K[blk] if pool == "k" else self.V[blk]).astype(np.float64)

    def gather(self, table, L: int, start: int = 0):
        """K, V of positions start .. L-1 of one sequence, [H, L - start, D] fp64, read token by
        token through its block table."""
        K = np.zeros((self.H, L - start, self.D))
        V = np.zeros((self.H, L - start, self.D))
        cache = {}
        for t in range(start, L):
            blk, off = int(table[t // BS]), t % BS
            if blk < 0:
                raise ValueError(f"position {t} lies in a dropped block")
            if blk not in cache:
                cache[blk] = (self.values("k", blk), self.values("v", blk))
            K[:, t - start, :] = cache[blk][0][:, off, :]
            V[:, t - start, :] = cache[blk][1][:, off, :]
        return K, V

    def prefill(self, q, q_start, tables, lens, scale) -> np.ndarray:
        """As ContigCache.prefill, the positions read through the block tables."""
        return _prefill(q, q_start, lens, scale, self.H,
                        lambda b, L: self.gather(tables[b], L))

    def decode(self, q, tables, lens, scale, heads=None, window: int = 0) -> np.ndarray:
        """q: [B, Hq, D] with Hq a multiple of the pool's H (query head hq reads key/value head
        kv_head_of(hq, Hq, H), as in grouped_decode); tables: [B, max_blocks]; lens[b]: attended
        length; window > 0: only positions window_start(lens[b], window) .. lens[b]-1 are
        attended (rolling window). Returns [B, Hq, D] (only the listed query heads are computed
        when `heads` is given; the rest stay 0)."""
        B, Hq = len(lens), q.shape[1]
        G = Hq // self.H
        if G * self.H != Hq:
            raise ValueError("query heads must be a multiple of the pool's heads")
        out = np.zeros((B, Hq, self.D))
        hs = range(Hq) if heads is None else heads
        for b in range(B):
            K, V = self.gather(tables[b], int(lens[b]), window_start(int(lens[b]), window))
            for h in hs:
                out[b, h] = decode_row(q[b, h], K[h // G], V[h // G], scale)
        return out


def _prefill(q, q_start, lens, scale, H, kv_of) -> np.ndarray:
    """Chunked prefill through a cache model: for each sequence, full_causal over its chunk
    ("LLM Inference Acceleration -- KV Cache", section 3.1: the chunk's K/V are written at
    start_pos, then rows attend positions 0 .. start_pos + i under triu(-inf, start_pos + 1))."""
    q = np.asarray(q)
    Hq = q.shape[1]
    out = np.zeros(q.shape, dtype=np.float64)
    for b in range(len(lens)):
        r0, r1 = int(q_start[b]), int(q_start[b + 1])
        n, L = r1 - r0, int(lens[b])
        if n == 0:
            continue
        K, V = kv_of(b, L)
        for hq in range(Hq):
            g = kv_head_of(hq, Hq, H)
            out[r0:r1, hq] = full_causal(q[r0:r1, hq], K[g], V[g], scale, start_pos=L - n)
    return out
