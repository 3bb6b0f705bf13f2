"""Python binding of libkvc: decode attention over a KV cache on AMD MI355X (gfx950).

Argument marshalling only: every step runs in libkvc (host block pool in C++, cache writes and
attention in HIP kernels). torch is used for device memory and streams. The library must have
been built (`python -m kv_cache_attention_kvc_amd.csrc.build`); importing works without it, but
the first call raises if libkvc.so is missing -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

__all__ = [
    "KvcError", "load_library", "library_path", "Pool", "PagedLayer",
    "F32", "F16", "E4M3", "I8", "BLOCK_SIZE", "workspace_bytes",
    "append_contig", "copy_blocks", "write_paged", "decode_attn_contig", "decode_attn_paged",
    "decode_partial_contig", "decode_partial_paged", "decode_merge", "new_workspace", "EXPORTS",
    "append_decode_contig", "append_decode_paged", "append_decode_partial_contig",
    "append_decode_partial_paged", "gqa_workspace_bytes", "new_gqa_workspace",
    "decode_gqa_contig", "decode_gqa_paged", "decode_gqa_partial_contig",
    "decode_gqa_partial_paged", "decode_gqa_merge", "decode_window_contig", "decode_window_paged",
    "decode_window_partial_contig", "decode_window_partial_paged", "prefill_contig",
    "prefill_paged", "compress_blocks", "append_decode_gqa_contig", "append_decode_gqa_paged",
    "append_decode_gqa_partial_contig", "append_decode_gqa_partial_paged",
    "decode_attn_paged_noalloc", "read_pieces",
]

F32, F16, E4M3, I8 = 0, 1, 2, 3
BLOCK_SIZE = 16
_STATUS = {0: "KVC_OK", -1: "KVC_E_INVALID", -2: "KVC_E_OOM", -3: "KVC_E_NOSEQ",
           -4: "KVC_E_CAPACITY", -5: "KVC_E_UNSUPPORTED", -6: "KVC_E_HIP"}

# every symbol include/kvc.h declares
EXPORTS = [
    "kvc_status_str", "kvc_pool_create", "kvc_pool_destroy", "kvc_alloc", "kvc_append",
    "kvc_fork", "kvc_free", "kvc_slide", "kvc_block_table", "kvc_stats", "kvc_check",
    "kvc_append_contig",
    "kvc_copy_blocks", "kvc_write_paged", "kvc_decode_workspace_bytes", "kvc_decode_attn_contig",
    "kvc_decode_attn_paged", "kvc_decode_partial_contig", "kvc_decode_partial_paged",
    "kvc_decode_merge", "kvc_append_decode_contig", "kvc_append_decode_paged",
    "kvc_append_decode_partial_contig", "kvc_append_decode_partial_paged",
    "kvc_gqa_workspace_bytes", "kvc_decode_gqa_contig", "kvc_decode_gqa_paged",
    "kvc_decode_gqa_partial_contig", "kvc_decode_gqa_partial_paged", "kvc_decode_gqa_merge",
    "kvc_decode_window_contig", "kvc_decode_window_paged", "kvc_decode_window_partial_contig",
    "kvc_decode_window_partial_paged", "kvc_prefill_contig", "kvc_prefill_paged",
    "kvc_compress_blocks", "kvc_append_decode_gqa_contig", "kvc_append_decode_gqa_paged",
    "kvc_append_decode_gqa_partial_contig", "kvc_append_decode_gqa_partial_paged",
    "kvc_decode_attn_paged_noalloc", "kvc_read_pieces", "kvc_decode_merge_needed",
]


class KvcError(RuntimeError):
    def __init__(self, status: int, where: str = ""):
        self.status = status
        name = _STATUS.get(status, str(status))
        msg = _lib().kvc_status_str(status).decode() if _LIB is not None else name
        super().__init__(f"{where}: {name} ({msg})" if where else f"{name} ({msg})")


class PoolStats(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("used", ctypes.c_int32),
                ("free_blocks", ctypes.c_int32), ("shared", ctypes.c_int32),
                ("num_seqs", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("cow_copies", ctypes.c_int64), ("tokens", ctypes.c_int64),
                ("slots_logical", ctypes.c_int64)]


class _Layer(ctypes.Structure):
    _fields_ = [("kv_dtype", ctypes.c_int), ("num_blocks", ctypes.c_int32),
                ("num_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p),
                ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p)]


_LIB: Optional[ctypes.CDLL] = None
_P = ctypes.c_void_p
_I32, _I64, _F = ctypes.c_int32, ctypes.c_int64, ctypes.c_float
_PI32 = ctypes.POINTER(ctypes.c_int32)
_PI64 = ctypes.POINTER(ctypes.c_int64)


def library_path() -> str:
    return os.environ.get("KVC_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                     "libkvc.so")


def load_library() -> ctypes.CDLL:
    """Load libkvc.so and declare its signatures. Raises if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"libkvc.so not found at {path}; build it with "
                           "`python -m kv_cache_attention_kvc_amd.csrc.build`")
    lib = ctypes.CDLL(path)
    sig = {
        "kvc_status_str": (ctypes.c_char_p, [ctypes.c_int]),
        "kvc_pool_create": (ctypes.c_int, [_I32, _I32, _I32, _P, ctypes.POINTER(_P)]),
        "kvc_pool_destroy": (None, [_P]),
        "kvc_alloc": (ctypes.c_int, [_P, _PI32]),
        "kvc_append": (ctypes.c_int, [_P, _P, _I32, _I32, _P, _P, _P, _I32, _PI32]),
        "kvc_fork": (ctypes.c_int, [_P, _I32, _PI32]),
        "kvc_free": (ctypes.c_int, [_P, _I32]),
        "kvc_slide": (ctypes.c_int, [_P, _P, _I32, _I32, _PI32]),
        "kvc_block_table": (ctypes.c_int, [_P, _P, _I32, _P, _P]),
        "kvc_stats": (ctypes.c_int, [_P, ctypes.POINTER(PoolStats)]),
        "kvc_check": (ctypes.c_int, [_P]),
        "kvc_append_contig": (ctypes.c_int, [_P, _P, ctypes.c_int, _I32, _I32, _I32, _I32, _P,
                                             _I32, _P, _P, _P]),
        "kvc_copy_blocks": (ctypes.c_int, [ctypes.POINTER(_Layer), _P, _P, _I32, _P]),
        "kvc_write_paged": (ctypes.c_int, [ctypes.POINTER(_Layer), _P, _I32, _P, _P, ctypes.c_int,
                                           _P]),
        "kvc_compress_blocks": (ctypes.c_int, [ctypes.POINTER(_Layer), ctypes.POINTER(_Layer), _P,
                                               _P, _P, _I32, _P]),
        "kvc_decode_workspace_bytes": (ctypes.c_size_t, [_I32, _I32, _I32]),
        "kvc_decode_attn_contig": (ctypes.c_int, [_P, ctypes.c_int, _P, _P, ctypes.c_int, _P, _I32,
                                                  _I32, _I32, _I32, _I32, _F, _P, ctypes.c_int, _P,
                                                  ctypes.c_size_t, _P]),
        "kvc_decode_attn_paged": (ctypes.c_int, [_P, ctypes.c_int, ctypes.POINTER(_Layer), _P, _I32,
                                                 _P, _I32, _I32, _F, _P, ctypes.c_int, _P,
                                                 ctypes.c_size_t, _P]),
        "kvc_decode_attn_paged_noalloc": (ctypes.c_int, [_P, ctypes.c_int, ctypes.POINTER(_Layer),
                                                         _P, _I32, _P, _I32, _I32, _F, _P,
                                                         ctypes.c_int, _P]),
        "kvc_read_pieces": (ctypes.c_int, [_P, _P, _P, _I32, _I32, _I32, _P, ctypes.c_size_t,
                                           _P]),
        "kvc_decode_partial_contig": (ctypes.c_int, [_P, ctypes.c_int, _P, _P, ctypes.c_int, _P,
                                                     _I32, _I32, _I32, _I32, _I32, _F, _P,
                                                     ctypes.c_int, _P, ctypes.c_size_t, _P]),
        "kvc_decode_partial_paged": (ctypes.c_int, [_P, ctypes.c_int, ctypes.POINTER(_Layer), _P,
                                                    _I32, _P, _I32, _I32, _F, _P, ctypes.c_int, _P,
                                                    ctypes.c_size_t, _P]),
        "kvc_decode_merge": (ctypes.c_int, [_I32, _I32, _I32, _P, ctypes.c_int, _P,
                                            ctypes.c_size_t, _P]),
        "kvc_decode_merge_needed": (ctypes.c_int, [_I32, _I32, ctypes.c_int, ctypes.c_int, _I32,
                                                   _I32, _I32, _I32, _I32, _I32, _I32, _PI32]),
    }
    contig_append = [_P, ctypes.c_int, _P, _P, ctypes.c_int, _P, _P, _P, _I32, _I32, _I32, _I32,
                     _I32, _F, _P, ctypes.c_int, _P, ctypes.c_size_t, _P]
    paged_append = [_P, ctypes.c_int, ctypes.POINTER(_Layer), _P, _I32, _P, _P, _P, _I32, _I32,
                    _F, _P, ctypes.c_int, _P, ctypes.c_size_t, _P]
    for name in ("kvc_append_decode_contig", "kvc_append_decode_partial_contig"):
        sig[name] = (ctypes.c_int, contig_append)
    for name in ("kvc_append_decode_paged", "kvc_append_decode_partial_paged"):
        sig[name] = (ctypes.c_int, paged_append)
    contig_gqa = [_P, ctypes.c_int, _I32, _P, _P, ctypes.c_int, _P, _I32, _I32, _I32, _I32, _I32,
                  _F, _P, ctypes.c_int, _P, ctypes.c_size_t, _P]
    paged_gqa = [_P, ctypes.c_int, _I32, ctypes.POINTER(_Layer), _P, _I32, _P, _I32, _I32, _F, _P,
                 ctypes.c_int, _P, ctypes.c_size_t, _P]
    for name in ("kvc_decode_gqa_contig", "kvc_decode_gqa_partial_contig"):
        sig[name] = (ctypes.c_int, contig_gqa)
    for name in ("kvc_decode_gqa_paged", "kvc_decode_gqa_partial_paged"):
        sig[name] = (ctypes.c_int, paged_gqa)
    sig["kvc_gqa_workspace_bytes"] = (ctypes.c_size_t, [_I32, _I32, _I32, _I32])
    contig_gqa_append = contig_gqa[:7] + [_P, _P] + contig_gqa[7:]   # k_new, v_new after lens
    paged_gqa_append = paged_gqa[:7] + [_P, _P] + paged_gqa[7:]
    for name in ("kvc_append_decode_gqa_contig", "kvc_append_decode_gqa_partial_contig"):
        sig[name] = (ctypes.c_int, contig_gqa_append)
    for name in ("kvc_append_decode_gqa_paged", "kvc_append_decode_gqa_partial_paged"):
        sig[name] = (ctypes.c_int, paged_gqa_append)
    contig_win = contig_gqa[:12] + [_I32] + contig_gqa[12:]   # window after max_ctx
    paged_win = paged_gqa[:9] + [_I32] + paged_gqa[9:]
    for name in ("kvc_decode_window_contig", "kvc_decode_window_partial_contig"):
        sig[name] = (ctypes.c_int, contig_win)
    for name in ("kvc_decode_window_paged", "kvc_decode_window_partial_paged"):
        sig[name] = (ctypes.c_int, paged_win)
    sig["kvc_prefill_contig"] = (ctypes.c_int, [_P, ctypes.c_int, _I32, _P, _P, ctypes.c_int, _P,
                                                _P, _I32, _I32, _I32, _I32, _I32, _F, _P,
                                                ctypes.c_int, _P])
    sig["kvc_prefill_paged"] = (ctypes.c_int, [_P, ctypes.c_int, _I32, ctypes.POINTER(_Layer), _P,
                                               _I32, _P, _P, _I32, _I32, _F, _P, ctypes.c_int,
                                               _P])
    sig["kvc_decode_gqa_merge"] = (ctypes.c_int, [_I32, _I32, _I32, _I32, _P, ctypes.c_int, _P,
                                                  ctypes.c_size_t, _P])
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = lib
    return lib


def _lib() -> ctypes.CDLL:
    return _LIB if _LIB is not None else load_library()


def _check(status: int, where: str) -> None:
    if status != 0:
        raise KvcError(status, where)


# ---------------------------------------------------------------------------------------------
# Host block pool
# ---------------------------------------------------------------------------------------------
class Pool:
    """Host-side block pool: first fit, refcounts, fork, copy-on-write, rolling-window slide
    (libkvc C++)."""

    def __init__(self, num_blocks: int, max_blocks_per_seq: int, order=None,
                 block_size: int = BLOCK_SIZE):
        lib = _lib()
        self.num_blocks = int(num_blocks)
        self.max_blocks_per_seq = int(max_blocks_per_seq)
        h = _P()
        if order is not None:
            self._order = np.ascontiguousarray(order, dtype=np.int32)
            optr = self._order.ctypes.data
        else:
            optr = None
        _check(lib.kvc_pool_create(num_blocks, block_size, max_blocks_per_seq, optr,
                                   ctypes.byref(h)), "kvc_pool_create")
        self._h = h

    def close(self) -> None:
        if getattr(self, "_h", None):
            _lib().kvc_pool_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def alloc(self) -> int:
        s = ctypes.c_int32()
        _check(_lib().kvc_alloc(self._h, ctypes.byref(s)), "kvc_alloc")
        return s.value

    def append(self, seqs: Sequence[int], n_tokens: int):
        """Returns (slots int64[n_seqs*n_tokens], cow_src int32[n], cow_dst int32[n])."""
        seqs = np.ascontiguousarray(seqs, dtype=np.int32)
        n = len(seqs)
        slots = np.empty(max(1, n * n_tokens), dtype=np.int64)
        src = np.empty(max(1, n), dtype=np.int32)
        dst = np.empty(max(1, n), dtype=np.int32)
        ncow = ctypes.c_int32()
        _check(_lib().kvc_append(self._h, seqs.ctypes.data, n, n_tokens, slots.ctypes.data,
                                 src.ctypes.data, dst.ctypes.data, max(1, n),
                                 ctypes.byref(ncow)), "kvc_append")
        k = ncow.value
        return slots[:n * n_tokens], src[:k].copy(), dst[:k].copy()

    def fork(self, parent: int) -> int:
        c = ctypes.c_int32()
        _check(_lib().kvc_fork(self._h, parent, ctypes.byref(c)), "kvc_fork")
        return c.value

    def free(self, seq: int) -> None:
        _check(_lib().kvc_free(self._h, seq), "kvc_free")

    def slide(self, seqs: Sequence[int], window: int) -> int:
        """Rolling window: drop from each sequence the blocks wholly before its last `window`
        positions (table entries become -1). Returns the number of entries dropped."""
        seqs = np.ascontiguousarray(seqs, dtype=np.int32)
        n = ctypes.c_int32()
        _check(_lib().kvc_slide(self._h, seqs.ctypes.data, len(seqs), int(window),
                                ctypes.byref(n)), "kvc_slide")
        return n.value

    def block_table(self, seqs: Sequence[int], out_tables=None, out_lens=None):
        """Tables [n, max_blocks_per_seq] (-1 padded) and lengths [n], int32. Optional output
        arrays (e.g. pinned host tensors' numpy views) are filled in place."""
        seqs = np.ascontiguousarray(seqs, dtype=np.int32)
        n = len(seqs)
        t = out_tables if out_tables is not None else np.empty((n, self.max_blocks_per_seq),
                                                               dtype=np.int32)
        ln = out_lens if out_lens is not None else np.empty(n, dtype=np.int32)
        assert t.dtype == np.int32 and t.flags.c_contiguous and t.shape == (n, self.max_blocks_per_seq)
        assert ln.dtype == np.int32 and ln.shape == (n,)
        _check(_lib().kvc_block_table(self._h, seqs.ctypes.data, n, t.ctypes.data, ln.ctypes.data),
               "kvc_block_table")
        return t, ln

    def stats(self) -> dict:
        st = PoolStats()
        _check(_lib().kvc_stats(self._h, ctypes.byref(st)), "kvc_stats")
        return {f: getattr(st, f) for f, _ in PoolStats._fields_ if f != "reserved"}

    def check(self) -> None:
        _check(_lib().kvc_check(self._h), "kvc_check")


# ---------------------------------------------------------------------------------------------
# Device side (torch tensors on the current device; launches on the current torch stream)
# ---------------------------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.float16:
        return F16
    if t.dtype == torch.uint8:
        return E4M3
    if t.dtype == torch.int8:
        return I8
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t) -> int:
    if not t.is_cuda:
        raise ValueError("tensor must live in device memory")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _ptr_i32(t) -> int:
    """Device pointer of an int32 index tensor (block tables, lengths, positions, block ids)."""
    if t.dtype != _torch().int32:
        raise ValueError(f"index tensor must be int32, got {t.dtype}")
    return _ptr(t)


def _ptr_i64(t) -> int:
    """Device pointer of an int64 slot tensor."""
    if t.dtype != _torch().int64:
        raise ValueError(f"slot tensor must be int64, got {t.dtype}")
    return _ptr(t)


def _stream(stream) -> int:
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


@dataclass
class PagedLayer:
    """One layer of a paged cache: pools [num_blocks, H, 16, D] (float32/float16, or uint8 holding
    e4m3 codes / int8 codes, with float32 scales [num_blocks] for K and V)."""
    k_pool: object
    v_pool: object
    k_scale: object = None
    v_scale: object = None

    @staticmethod
    def empty(num_blocks: int, heads: int, head_dim: int, dtype: str, device="cuda", fill=None):
        torch = _torch()
        td = {"f32": torch.float32, "f16": torch.float16, "e4m3": torch.uint8,
              "i8": torch.int8}[dtype]
        shape = (num_blocks, heads, BLOCK_SIZE, head_dim)
        if dtype == "e4m3" and fill is not None:
            fill = 0x7F if fill != fill else int(fill)     # NaN -> the e4m3 NaN code
        if dtype == "i8" and fill is not None:
            fill = -128 if fill != fill else int(fill)     # NaN -> the never-written int8 code
        if fill is None:
            k = torch.zeros(shape, dtype=td, device=device)
            v = torch.zeros(shape, dtype=td, device=device)
        else:
            k = torch.full(shape, fill, dtype=td, device=device)
            v = torch.full(shape, fill, dtype=td, device=device)
        ks = vs = None
        if dtype in ("e4m3", "i8"):
            ks = torch.zeros(num_blocks, dtype=torch.float32, device=device)
            vs = torch.zeros(num_blocks, dtype=torch.float32, device=device)
        return PagedLayer(k, v, ks, vs)

    @property
    def num_blocks(self) -> int:
        return self.k_pool.shape[0]

    @property
    def heads(self) -> int:
        return self.k_pool.shape[1]

    @property
    def head_dim(self) -> int:
        return self.k_pool.shape[3]

    def struct(self) -> _Layer:
        key = (self.k_pool.data_ptr(), self.v_pool.data_ptr(),
               None if self.k_scale is None else self.k_scale.data_ptr(),
               None if self.v_scale is None else self.v_scale.data_ptr(), tuple(self.k_pool.shape))
        cached = getattr(self, "_cached", None)
        if cached is not None and cached[0] == key:
            return cached[1]
        if tuple(self.k_pool.shape) != tuple(self.v_pool.shape) or self.k_pool.dim() != 4 \
                or self.k_pool.shape[2] != BLOCK_SIZE:
            raise ValueError("pools must be [num_blocks, H, 16, D] and alike")
        code = _dtype_code(self.k_pool)
        s = _Layer(code, self.num_blocks, self.heads, self.head_dim, _ptr(self.k_pool),
                   _ptr(self.v_pool), None, None)
        if code in (E4M3, I8):
            s.k_scale = _ptr(self.k_scale)
            s.v_scale = _ptr(self.v_scale)
        self._cached = (key, s)
        return s


def workspace_bytes(B: int, H: int, D: int) -> int:
    return int(_lib().kvc_decode_workspace_bytes(B, H, D))


def new_workspace(B: int, H: int, D: int, device="cuda"):
    """A decode workspace for batches of up to B sequences (no initialisation needed)."""
    torch = _torch()
    return torch.empty(workspace_bytes(B, H, D), dtype=torch.uint8, device=device)


def _workspace(B, H, D, ws, device):
    return new_workspace(B, H, D, device) if ws is None else ws   # libkvc checks the size


def append_contig(k_cache, v_cache, pos, k_new, v_new, stream=None) -> None:
    """K[b,h,pos[b]+t,:] = k_new[b,t,h,:] (k_cache [B,H,S_max,D], k_new [B,n,H,D], pos int32[B])."""
    B, H, S, D = k_cache.shape
    if k_new.shape[0] != B or k_new.shape[2] != H or k_new.shape[3] != D:
        raise ValueError("k_new must be [B, n, H, D]")
    if k_new.dtype != k_cache.dtype or v_new.dtype != v_cache.dtype:
        raise ValueError("new K/V must have the cache dtype")
    _check(_lib().kvc_append_contig(_ptr(k_cache), _ptr(v_cache), _dtype_code(k_cache), B, H, S,
                                    D, _ptr_i32(pos), k_new.shape[1], _ptr(k_new), _ptr(v_new),
                                    _stream(stream)), "kvc_append_contig")


def copy_blocks(layer: PagedLayer, src, dst, stream=None) -> None:
    n = int(src.numel())
    if n == 0:
        return
    st = layer.struct()
    _check(_lib().kvc_copy_blocks(ctypes.byref(st), _ptr_i32(src), _ptr_i32(dst), n, _stream(stream)),
           "kvc_copy_blocks")


def write_paged(layer: PagedLayer, slots, k_new, v_new, stream=None) -> None:
    """Store k_new/v_new [n, H, D] at int64 slots[n] (fp8 pools quantise per block)."""
    n = int(slots.numel())
    if n == 0:
        return
    if tuple(k_new.shape) != (n, layer.heads, layer.head_dim) or k_new.shape != v_new.shape:
        raise ValueError("k_new/v_new must be [n, H, D]")
    st = layer.struct()
    _check(_lib().kvc_write_paged(ctypes.byref(st), _ptr_i64(slots), n, _ptr(k_new), _ptr(v_new),
                                  _dtype_code(k_new), _stream(stream)), "kvc_write_paged")


def compress_blocks(src: PagedLayer, dst: PagedLayer, src_ids, dst_ids, n_valid=None,
                    stream=None) -> None:
    """Re-encode blocks src_ids of a 16-bit (or fp32) layer into blocks dst_ids of an 8-bit
    layer (int32 device tensors of equal length); n_valid: int32 slots per block that hold
    positions (None: all 16). Each destination block gets a fresh per-block scale."""
    n = int(src_ids.numel())
    if int(dst_ids.numel()) != n or (n_valid is not None and int(n_valid.numel()) != n):
        raise ValueError("src_ids, dst_ids and n_valid must have one entry per block pair")
    if n == 0:
        return
    s1, s2 = src.struct(), dst.struct()
    _check(_lib().kvc_compress_blocks(ctypes.byref(s1), ctypes.byref(s2), _ptr_i32(src_ids),
                                      _ptr_i32(dst_ids), None if n_valid is None else _ptr_i32(n_valid),
                                      n, _stream(stream)), "kvc_compress_blocks")


def _out_for(q, out):
    """The output tensor: a new one like q, or the caller's, which must have q's shape and an
    fp32 or fp16 dtype (the library cannot see the size of device arrays)."""
    torch = _torch()
    if out is None:
        return torch.empty_like(q)
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError(f"out must have q's shape {tuple(q.shape)}, got {tuple(out.shape)}")
    if out.dtype not in (torch.float32, torch.float16):
        raise ValueError(f"out must be float32 or float16, got {out.dtype}")
    return out


def _check_lens(ctx_lens, B: int) -> None:
    """ctx_lens holds one int32 length per sequence."""
    if ctx_lens.dim() != 1 or int(ctx_lens.numel()) != B:
        raise ValueError(f"ctx_lens must be int32[{B}], got shape {tuple(ctx_lens.shape)}")


def _check_tables(block_tables, B: int) -> None:
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [B, max_blocks]")


def _check_q_start(q_start, B: int) -> None:
    if q_start.dim() != 1 or int(q_start.numel()) != B + 1:
        raise ValueError(f"q_start must be int32[{B + 1}], got shape {tuple(q_start.shape)}")


def _check_merge_out(out, rows: int, D: int) -> None:
    """The merge writes rows x D elements of out (fp32 or fp16)."""
    torch = _torch()
    if int(out.numel()) != rows * D or out.dtype not in (torch.float32, torch.float16):
        raise ValueError(f"out must hold {rows} x {D} float32/float16 elements, got "
                         f"{tuple(out.shape)} {out.dtype}")


def _check_q_mha(q, B: int, H: int, D: int) -> None:
    if tuple(q.shape) != (B, H, D):
        raise ValueError(f"q must be [B, H, D] = {(B, H, D)}, got {tuple(q.shape)}")


def decode_partial_contig(q, k_cache, v_cache, ctx_lens, max_ctx, scale=None, out=None,
                          workspace=None, stream=None):
    """Pass 1 only (see decode_attn_contig); returns (out, workspace) for decode_merge."""
    B, H, S, D = k_cache.shape
    _check_q_mha(q, B, H, D)
    _check_lens(ctx_lens, B)
    out = _out_for(q, out)
    ws = _workspace(B, H, D, workspace, q.device)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    _check(_lib().kvc_decode_partial_contig(
        _ptr(q), _dtype_code(q), _ptr(k_cache), _ptr(v_cache), _dtype_code(k_cache), _ptr_i32(ctx_lens),
        B, H, S, D, int(max_ctx), float(scale), _ptr(out), _dtype_code(out), _ptr(ws),
        ws.numel(), _stream(stream)), "kvc_decode_partial_contig")
    return out, ws


def decode_partial_paged(q, layer: PagedLayer, block_tables, ctx_lens, max_ctx, scale=None,
                         out=None, workspace=None, stream=None):
    """Pass 1 only (see decode_attn_paged); returns (out, workspace) for decode_merge."""
    B = q.shape[0]
    _check_q_mha(q, B, layer.heads, layer.head_dim)
    _check_tables(block_tables, B)
    _check_lens(ctx_lens, B)
    out = _out_for(q, out)
    ws = _workspace(B, layer.heads, layer.head_dim, workspace, q.device)
    scale = 1.0 / math.sqrt(layer.head_dim) if scale is None else scale
    st = layer.struct()
    _check(_lib().kvc_decode_partial_paged(
        _ptr(q), _dtype_code(q), ctypes.byref(st), _ptr_i32(block_tables), block_tables.shape[1],
        _ptr_i32(ctx_lens), B, int(max_ctx), float(scale), _ptr(out), _dtype_code(out), _ptr(ws),
        ws.numel(), _stream(stream)), "kvc_decode_partial_paged")
    return out, ws


def decode_merge(B, H, D, out, workspace, stream=None):
    """Pass 2: combine the split sequence-heads that pass 1 left in `workspace`."""
    _check_merge_out(out, B * H, D)
    _check(_lib().kvc_decode_merge(B, H, D, _ptr(out), _dtype_code(out), _ptr(workspace),
                                   workspace.numel(), _stream(stream)), "kvc_decode_merge")
    return out


_DTYPE_NAMES = {"f32": F32, "f16": F16, "e4m3": E4M3, "i8": I8}


def decode_merge_needed(paged: bool, q_dtype: str, kv_dtype: str, B: int, H: int, D: int,
                        cap: int, max_ctx: int, G: int = 1, window: int = 0,
                        append: bool = False) -> bool:
    """Whether pass 1 of these sizes leaves records for the merge (kvc_decode_merge_needed);
    False means it finishes every row itself and the merge launch can be skipped. dtypes by
    name ("f32", "f16", "e4m3", "i8"); cap: S_max or 16 * max_blocks_per_seq."""
    needed = ctypes.c_int32(0)
    _check(_lib().kvc_decode_merge_needed(int(bool(paged)), int(bool(append)),
                                          _DTYPE_NAMES[q_dtype], _DTYPE_NAMES[kv_dtype], int(B),
                                          int(H), int(G), int(D), int(cap), int(max_ctx),
                                          int(window), ctypes.byref(needed)),
           "kvc_decode_merge_needed")
    return needed.value != 0


def decode_attn_contig(q, k_cache, v_cache, ctx_lens, max_ctx, scale=None, out=None,
                       workspace=None, stream=None):
    """Single-query attention over a contiguous cache: q [B,H,D], caches [B,H,S_max,D],
    ctx_lens int32[B] on the device. Returns out [B,H,D] (q's dtype unless `out` is given)."""
    B, H, S, D = k_cache.shape
    _check_q_mha(q, B, H, D)
    _check_lens(ctx_lens, B)
    out = _out_for(q, out)
    ws = _workspace(B, H, D, workspace, q.device)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    _check(_lib().kvc_decode_attn_contig(
        _ptr(q), _dtype_code(q), _ptr(k_cache), _ptr(v_cache), _dtype_code(k_cache), _ptr_i32(ctx_lens),
        B, H, S, D, int(max_ctx), float(scale), _ptr(out), _dtype_code(out), _ptr(ws),
        ws.numel(), _stream(stream)), "kvc_decode_attn_contig")
    return out


def decode_attn_paged(q, layer: PagedLayer, block_tables, ctx_lens, max_ctx, scale=None,
                      out=None, workspace=None, stream=None):
    """Single-query attention over a paged cache: q [B,H,D], block_tables int32 [B, max_blocks]
    and ctx_lens int32[B] on the device. Returns out [B,H,D]."""
    B = q.shape[0]
    _check_q_mha(q, B, layer.heads, layer.head_dim)
    _check_tables(block_tables, B)
    _check_lens(ctx_lens, B)
    out = _out_for(q, out)
    ws = _workspace(B, layer.heads, layer.head_dim, workspace, q.device)
    scale = 1.0 / math.sqrt(layer.head_dim) if scale is None else scale
    st = layer.struct()
    _check(_lib().kvc_decode_attn_paged(
        _ptr(q), _dtype_code(q), ctypes.byref(st), _ptr_i32(block_tables), block_tables.shape[1],
        _ptr_i32(ctx_lens), B, int(max_ctx), float(scale), _ptr(out), _dtype_code(out), _ptr(ws),
        ws.numel(), _stream(stream)), "kvc_decode_attn_paged")
    return out


def decode_attn_paged_noalloc(q, layer: PagedLayer, block_tables, ctx_lens, max_ctx, scale=None,
                              out=None, stream=None):
    """decode_attn_paged with the library's own static workspace (kvc_decode_attn_paged_noalloc:
    no device allocation in the call, B <= 4096). Pass `out` to allocate nothing at all. Calls
    that may overlap in time on one GPU share that workspace and must be serialised."""
    B = q.shape[0]
    _check_q_mha(q, B, layer.heads, layer.head_dim)
    _check_tables(block_tables, B)
    _check_lens(ctx_lens, B)
    out = _out_for(q, out)
    scale = 1.0 / math.sqrt(layer.head_dim) if scale is None else scale
    st = layer.struct()
    _check(_lib().kvc_decode_attn_paged_noalloc(
        _ptr(q), _dtype_code(q), ctypes.byref(st), _ptr_i32(block_tables), block_tables.shape[1],
        _ptr_i32(ctx_lens), B, int(max_ctx), float(scale), _ptr(out), _dtype_code(out),
        _stream(stream)), "kvc_decode_attn_paged_noalloc")
    return out


def _check_new(k_new, v_new, B, H, D, dtype):
    if tuple(k_new.shape) != (B, H, D) or tuple(v_new.shape) != (B, H, D):
        raise ValueError("k_new/v_new must be [B, H, D]")
    if k_new.dtype != dtype or v_new.dtype != dtype:
        raise ValueError("k_new/v_new must have the cache dtype")


def _append_contig_call(name, q, k_cache, v_cache, ctx_lens, k_new, v_new, max_ctx, scale, out,
                        workspace, stream):
    B, H, S, D = k_cache.shape
    _check_q_mha(q, B, H, D)
    _check_lens(ctx_lens, B)
    _check_new(k_new, v_new, B, H, D, k_cache.dtype)
    out = _out_for(q, out)
    ws = _workspace(B, H, D, workspace, q.device)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    _check(getattr(_lib(), name)(
        _ptr(q), _dtype_code(q), _ptr(k_cache), _ptr(v_cache), _dtype_code(k_cache),
        _ptr_i32(ctx_lens), _ptr(k_new), _ptr(v_new), B, H, S, D, int(max_ctx), float(scale),
        _ptr(out), _dtype_code(out), _ptr(ws), ws.numel(), _stream(stream)), name)
    return out, ws


def _append_paged_call(name, q, layer, block_tables, ctx_lens, k_new, v_new, max_ctx, scale, out,
                       workspace, stream):
    B = q.shape[0]
    _check_q_mha(q, B, layer.heads, layer.head_dim)
    _check_tables(block_tables, B)
    _check_lens(ctx_lens, B)
    _check_new(k_new, v_new, B, layer.heads, layer.head_dim, layer.k_pool.dtype)
    out = _out_for(q, out)
    ws = _workspace(B, layer.heads, layer.head_dim, workspace, q.device)
    scale = 1.0 / math.sqrt(layer.head_dim) if scale is None else scale
    st = layer.struct()
    _check(getattr(_lib(), name)(
        _ptr(q), _dtype_code(q), ctypes.byref(st), _ptr_i32(block_tables), block_tables.shape[1],
        _ptr_i32(ctx_lens), _ptr(k_new), _ptr(v_new), B, int(max_ctx), float(scale), _ptr(out),
        _dtype_code(out), _ptr(ws), ws.numel(), _stream(stream)), name)
    return out, ws


def append_decode_contig(q, k_cache, v_cache, ctx_lens, k_new, v_new, max_ctx, scale=None,
                         out=None, workspace=None, stream=None):
    """Store k_new/v_new [B,H,D] at position ctx_lens[b]-1 of the contiguous cache and attend
    over positions [0, ctx_lens[b]) in the same pass. Returns out [B,H,D]."""
    return _append_contig_call("kvc_append_decode_contig", q, k_cache, v_cache, ctx_lens, k_new,
                               v_new, max_ctx, scale, out, workspace, stream)[0]


def append_decode_partial_contig(q, k_cache, v_cache, ctx_lens, k_new, v_new, max_ctx,
                                 scale=None, out=None, workspace=None, stream=None):
    """Pass 1 of append_decode_contig; returns (out, workspace) for decode_merge."""
    return _append_contig_call("kvc_append_decode_partial_contig", q, k_cache, v_cache, ctx_lens,
                               k_new, v_new, max_ctx, scale, out, workspace, stream)


def append_decode_paged(q, layer: PagedLayer, block_tables, ctx_lens, k_new, v_new, max_ctx,
                        scale=None, out=None, workspace=None, stream=None):
    """Store k_new/v_new [B,H,D] at position ctx_lens[b]-1 of each sequence's blocks (after the
    pool's append and its copy-on-write copies) and attend in the same pass. Returns out."""
    return _append_paged_call("kvc_append_decode_paged", q, layer, block_tables, ctx_lens, k_new,
                              v_new, max_ctx, scale, out, workspace, stream)[0]


def append_decode_partial_paged(q, layer: PagedLayer, block_tables, ctx_lens, k_new, v_new,
                                max_ctx, scale=None, out=None, workspace=None, stream=None):
    """Pass 1 of append_decode_paged; returns (out, workspace) for decode_merge."""
    return _append_paged_call("kvc_append_decode_partial_paged", q, layer, block_tables, ctx_lens,
                              k_new, v_new, max_ctx, scale, out, workspace, stream)


# ---- shared key/value heads (MQA / GQA) ----------------------------------------------------
def gqa_workspace_bytes(B: int, H_kv: int, G: int, D: int) -> int:
    return int(_lib().kvc_gqa_workspace_bytes(B, H_kv, G, D))


def new_gqa_workspace(B: int, H_kv: int, G: int, D: int, device="cuda"):
    """A workspace for grouped-query decode of up to B sequences (no initialisation needed)."""
    torch = _torch()
    return torch.empty(gqa_workspace_bytes(B, H_kv, G, D), dtype=torch.uint8, device=device)


def _gqa_group(q, H_kv):
    Hq = q.shape[1]
    if Hq % H_kv:
        raise ValueError("q heads must be a multiple of the cache's heads")
    return Hq // H_kv


def _gqa_contig_call(name, q, k_cache, v_cache, ctx_lens, max_ctx, scale, out, workspace, stream):
    B, H, S, D = k_cache.shape
    if q.dim() != 3 or q.shape[0] != B or q.shape[2] != D:
        raise ValueError("q must be [B, H_kv*G, D]")
    G = _gqa_group(q, H)
    _check_lens(ctx_lens, B)
    out = _out_for(q, out)
    ws = new_gqa_workspace(B, H, G, D, q.device) if workspace is None else workspace
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    _check(getattr(_lib(), name)(
        _ptr(q), _dtype_code(q), G, _ptr(k_cache), _ptr(v_cache), _dtype_code(k_cache),
        _ptr_i32(ctx_lens), B, H, S, D, int(max_ctx), float(scale), _ptr(out), _dtype_code(out),
        _ptr(ws), ws.numel(), _stream(stream)), name)
    return out, ws


def _gqa_paged_call(name, q, layer, block_tables, ctx_lens, max_ctx, scale, out, workspace,
                    stream):
    B = q.shape[0]
    if q.dim() != 3 or q.shape[2] != layer.head_dim:
        raise ValueError("q must be [B, H_kv*G, D]")
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [B, max_blocks]")
    G = _gqa_group(q, layer.heads)
    _check_lens(ctx_lens, B)
    out = _out_for(q, out)
    ws = (new_gqa_workspace(B, layer.heads, G, layer.head_dim, q.device) if workspace is None
          else workspace)
    scale = 1.0 / math.sqrt(layer.head_dim) if scale is None else scale
    st = layer.struct()
    _check(getattr(_lib(), name)(
        _ptr(q), _dtype_code(q), G, ctypes.byref(st), _ptr_i32(block_tables), block_tables.shape[1],
        _ptr_i32(ctx_lens), B, int(max_ctx), float(scale), _ptr(out), _dtype_code(out), _ptr(ws),
        ws.numel(), _stream(stream)), name)
    return out, ws


def decode_gqa_contig(q, k_cache, v_cache, ctx_lens, max_ctx, scale=None, out=None,
                      workspace=None, stream=None):
    """Grouped-query decode over a contiguous cache: q [B, H_kv*G, D], caches
    [B, H_kv, S_max, D]; query head hq reads K/V head hq // G. Returns out [B, H_kv*G, D]."""
    return _gqa_contig_call("kvc_decode_gqa_contig", q, k_cache, v_cache, ctx_lens, max_ctx,
                            scale, out, workspace, stream)[0]


def decode_gqa_partial_contig(q, k_cache, v_cache, ctx_lens, max_ctx, scale=None, out=None,
                              workspace=None, stream=None):
    """Pass 1 of decode_gqa_contig; returns (out, workspace) for decode_gqa_merge."""
    return _gqa_contig_call("kvc_decode_gqa_partial_contig", q, k_cache, v_cache, ctx_lens,
                            max_ctx, scale, out, workspace, stream)


def decode_gqa_paged(q, layer: PagedLayer, block_tables, ctx_lens, max_ctx, scale=None, out=None,
                     workspace=None, stream=None):
    """Grouped-query decode over a paged cache whose layer holds the K/V heads. q is
    [B, H_kv*G, D]. Returns out [B, H_kv*G, D]."""
    return _gqa_paged_call("kvc_decode_gqa_paged", q, layer, block_tables, ctx_lens, max_ctx,
                           scale, out, workspace, stream)[0]


def decode_gqa_partial_paged(q, layer: PagedLayer, block_tables, ctx_lens, max_ctx, scale=None,
                             out=None, workspace=None, stream=None):
    """Pass 1 of decode_gqa_paged; returns (out, workspace) for decode_gqa_merge."""
    return _gqa_paged_call("kvc_decode_gqa_partial_paged", q, layer, block_tables, ctx_lens,
                           max_ctx, scale, out, workspace, stream)


def decode_gqa_merge(B, H_kv, G, D, out, workspace, stream=None):
    """Pass 2 of grouped-query decode."""
    _check_merge_out(out, B * H_kv * G, D)
    _check(_lib().kvc_decode_gqa_merge(B, H_kv, G, D, _ptr(out), _dtype_code(out),
                                       _ptr(workspace), workspace.numel(), _stream(stream)),
           "kvc_decode_gqa_merge")
    return out


def _append_gqa_contig_call(name, q, k_cache, v_cache, ctx_lens, k_new, v_new, max_ctx, scale,
                            out, workspace, stream):
    B, H, S, D = k_cache.shape
    if q.dim() != 3 or q.shape[0] != B or q.shape[2] != D:
        raise ValueError("q must be [B, H_kv*G, D]")
    G = _gqa_group(q, H)
    _check_lens(ctx_lens, B)
    _check_new(k_new, v_new, B, H, D, k_cache.dtype)
    out = _out_for(q, out)
    ws = new_gqa_workspace(B, H, G, D, q.device) if workspace is None else workspace
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    _check(getattr(_lib(), name)(
        _ptr(q), _dtype_code(q), G, _ptr(k_cache), _ptr(v_cache), _dtype_code(k_cache),
        _ptr_i32(ctx_lens), _ptr(k_new), _ptr(v_new), B, H, S, D, int(max_ctx), float(scale),
        _ptr(out), _dtype_code(out), _ptr(ws), ws.numel(), _stream(stream)), name)
    return out, ws


def _append_gqa_paged_call(name, q, layer, block_tables, ctx_lens, k_new, v_new, max_ctx, scale,
                           out, workspace, stream):
    B = q.shape[0]
    if q.dim() != 3 or q.shape[2] != layer.head_dim:
        raise ValueError("q must be [B, H_kv*G, D]")
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [B, max_blocks]")
    G = _gqa_group(q, layer.heads)
    _check_lens(ctx_lens, B)
    _check_new(k_new, v_new, B, layer.heads, layer.head_dim, layer.k_pool.dtype)
    out = _out_for(q, out)
    ws = (new_gqa_workspace(B, layer.heads, G, layer.head_dim, q.device) if workspace is None
          else workspace)
    scale = 1.0 / math.sqrt(layer.head_dim) if scale is None else scale
    st = layer.struct()
    _check(getattr(_lib(), name)(
        _ptr(q), _dtype_code(q), G, ctypes.byref(st), _ptr_i32(block_tables), block_tables.shape[1],
        _ptr_i32(ctx_lens), _ptr(k_new), _ptr(v_new), B, int(max_ctx), float(scale), _ptr(out),
        _dtype_code(out), _ptr(ws), ws.numel(), _stream(stream)), name)
    return out, ws


def append_decode_gqa_contig(q, k_cache, v_cache, ctx_lens, k_new, v_new, max_ctx, scale=None,
                             out=None, workspace=None, stream=None):
    """Grouped-query append and attend: store k_new/v_new [B, H_kv, D] at position
    ctx_lens[b]-1 of the contiguous cache and attend with q [B, H_kv*G, D] in the same pass."""
    return _append_gqa_contig_call("kvc_append_decode_gqa_contig", q, k_cache, v_cache, ctx_lens,
                                   k_new, v_new, max_ctx, scale, out, workspace, stream)[0]


def append_decode_gqa_partial_contig(q, k_cache, v_cache, ctx_lens, k_new, v_new, max_ctx,
                                     scale=None, out=None, workspace=None, stream=None):
    """Pass 1 of append_decode_gqa_contig; returns (out, workspace) for decode_gqa_merge."""
    return _append_gqa_contig_call("kvc_append_decode_gqa_partial_contig", q, k_cache, v_cache,
                                   ctx_lens, k_new, v_new, max_ctx, scale, out, workspace, stream)


def append_decode_gqa_paged(q, layer: PagedLayer, block_tables, ctx_lens, k_new, v_new, max_ctx,
                            scale=None, out=None, workspace=None, stream=None):
    """Grouped-query append and attend over a paged cache: k_new/v_new [B, H_kv, D] go to
    position ctx_lens[b]-1 of each sequence's blocks; q is [B, H_kv*G, D]. Returns out."""
    return _append_gqa_paged_call("kvc_append_decode_gqa_paged", q, layer, block_tables, ctx_lens,
                                  k_new, v_new, max_ctx, scale, out, workspace, stream)[0]


def append_decode_gqa_partial_paged(q, layer: PagedLayer, block_tables, ctx_lens, k_new, v_new,
                                    max_ctx, scale=None, out=None, workspace=None, stream=None):
    """Pass 1 of append_decode_gqa_paged; returns (out, workspace) for decode_gqa_merge."""
    return _append_gqa_paged_call("kvc_append_decode_gqa_partial_paged", q, layer, block_tables,
                                  ctx_lens, k_new, v_new, max_ctx, scale, out, workspace, stream)


# ---- rolling window --------------------------------------------------------------------------
def _window_contig_call(name, q, k_cache, v_cache, ctx_lens, max_ctx, window, scale, out,
                        workspace, stream):
    B, H, S, D = k_cache.shape
    if q.dim() != 3 or q.shape[0] != B or q.shape[2] != D:
        raise ValueError("q must be [B, H_kv*G, D]")
    G = _gqa_group(q, H)
    _check_lens(ctx_lens, B)
    out = _out_for(q, out)
    ws = new_gqa_workspace(B, H, G, D, q.device) if workspace is None else workspace
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    _check(getattr(_lib(), name)(
        _ptr(q), _dtype_code(q), G, _ptr(k_cache), _ptr(v_cache), _dtype_code(k_cache),
        _ptr_i32(ctx_lens), B, H, S, D, int(max_ctx), int(window), float(scale), _ptr(out),
        _dtype_code(out), _ptr(ws), ws.numel(), _stream(stream)), name)
    return out, ws


def _window_paged_call(name, q, layer, block_tables, ctx_lens, max_ctx, window, scale, out,
                       workspace, stream):
    B = q.shape[0]
    if q.dim() != 3 or q.shape[2] != layer.head_dim:
        raise ValueError("q must be [B, H_kv*G, D]")
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [B, max_blocks]")
    G = _gqa_group(q, layer.heads)
    _check_lens(ctx_lens, B)
    out = _out_for(q, out)
    ws = (new_gqa_workspace(B, layer.heads, G, layer.head_dim, q.device) if workspace is None
          else workspace)
    scale = 1.0 / math.sqrt(layer.head_dim) if scale is None else scale
    st = layer.struct()
    _check(getattr(_lib(), name)(
        _ptr(q), _dtype_code(q), G, ctypes.byref(st), _ptr_i32(block_tables), block_tables.shape[1],
        _ptr_i32(ctx_lens), B, int(max_ctx), int(window), float(scale), _ptr(out), _dtype_code(out),
        _ptr(ws), ws.numel(), _stream(stream)), name)
    return out, ws


def decode_window_contig(q, k_cache, v_cache, ctx_lens, max_ctx, window, scale=None, out=None,
                         workspace=None, stream=None):
    """Rolling-window decode over a contiguous cache [B, H_kv, S_max, D]: sequence b attends its
    last `window` positions. q [B, H_kv*G, D] (G = 1: multi-head). Returns out."""
    return _window_contig_call("kvc_decode_window_contig", q, k_cache, v_cache, ctx_lens, max_ctx,
                               window, scale, out, workspace, stream)[0]


def decode_window_partial_contig(q, k_cache, v_cache, ctx_lens, max_ctx, window, scale=None,
                                 out=None, workspace=None, stream=None):
    """Pass 1 of decode_window_contig; returns (out, workspace) for decode_gqa_merge."""
    return _window_contig_call("kvc_decode_window_partial_contig", q, k_cache, v_cache, ctx_lens,
                               max_ctx, window, scale, out, workspace, stream)


def decode_window_paged(q, layer: PagedLayer, block_tables, ctx_lens, max_ctx, window, scale=None,
                        out=None, workspace=None, stream=None):
    """Rolling-window decode over a paged cache (tables may hold entries dropped by
    Pool.slide with the same window). q [B, H_kv*G, D]. Returns out."""
    return _window_paged_call("kvc_decode_window_paged", q, layer, block_tables, ctx_lens, max_ctx,
                              window, scale, out, workspace, stream)[0]


def decode_window_partial_paged(q, layer: PagedLayer, block_tables, ctx_lens, max_ctx, window,
                                scale=None, out=None, workspace=None, stream=None):
    """Pass 1 of decode_window_paged; returns (out, workspace) for decode_gqa_merge."""
    return _window_paged_call("kvc_decode_window_partial_paged", q, layer, block_tables, ctx_lens,
                              max_ctx, window, scale, out, workspace, stream)


# ---- chunked prefill ---------------------------------------------------------------------------
def prefill_contig(q, k_cache, v_cache, q_start, ctx_lens, scale=None, out=None, stream=None):
    """Causal attention of a chunk of new tokens per sequence over a contiguous cache
    [B, H_kv, S_max, D] that already holds them. q [total, H_kv*G, D] fp16; sequence b's rows
    are q_start[b] .. q_start[b+1]-1 (device int32 [B+1]), its last positions of ctx_lens[b]."""
    B, H, S, D = k_cache.shape
    if q.dim() != 3 or q.shape[2] != D:
        raise ValueError("q must be [total, H_kv*G, D]")
    G = _gqa_group(q, H)
    _check_lens(ctx_lens, B)
    _check_q_start(q_start, B)
    out = _out_for(q, out)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    _check(_lib().kvc_prefill_contig(
        _ptr(q), _dtype_code(q), G, _ptr(k_cache), _ptr(v_cache), _dtype_code(k_cache),
        _ptr_i32(q_start), _ptr_i32(ctx_lens), B, H, S, D, q.shape[0], float(scale), _ptr(out),
        _dtype_code(out), _stream(stream)), "kvc_prefill_contig")
    return out


def prefill_paged(q, layer: PagedLayer, block_tables, q_start, ctx_lens, scale=None, out=None,
                  stream=None):
    """As prefill_contig over a paged layer through the sequences' block tables [B, max_blocks]."""
    if q.dim() != 3 or q.shape[2] != layer.head_dim:
        raise ValueError("q must be [total, H_kv*G, D]")
    if block_tables.dim() != 2:
        raise ValueError("block_tables must be [B, max_blocks]")
    B = block_tables.shape[0]
    G = _gqa_group(q, layer.heads)
    _check_lens(ctx_lens, B)
    _check_q_start(q_start, B)
    out = _out_for(q, out)
    scale = 1.0 / math.sqrt(layer.head_dim) if scale is None else scale
    st = layer.struct()
    _check(_lib().kvc_prefill_paged(
        _ptr(q), _dtype_code(q), G, ctypes.byref(st), _ptr_i32(block_tables), block_tables.shape[1],
        _ptr_i32(q_start), _ptr_i32(ctx_lens), B, q.shape[0], float(scale), _ptr(out), _dtype_code(out),
        _stream(stream)), "kvc_prefill_paged")
    return out


# ---- measurement -------------------------------------------------------------------------------
def read_pieces(a, offsets, piece_bytes: int, waves_per_cu: int, sink, b=None, stream=None):
    """Read-ceiling probe (kvc_read_pieces): read piece_bytes at a + offsets[i] (and b +
    offsets[i]) for every entry of the int64 device tensor `offsets`, in contiguous runs per
    wavefront; `sink` is a device uint32 (int32) tensor of at least one word per wavefront. The
    offsets must keep every piece inside a (and b); the caller times the launch."""
    n = int(offsets.numel())
    nbytes = int(a.numel()) * a.element_size()
    if b is not None and int(b.numel()) * b.element_size() != nbytes:
        raise ValueError("a and b must have the same size")
    _check(_lib().kvc_read_pieces(_ptr(a), None if b is None else _ptr(b), _ptr_i64(offsets), n,
                                  int(piece_bytes), int(waves_per_cu), _ptr(sink),
                                  int(sink.numel()), _stream(stream)), "kvc_read_pieces")
