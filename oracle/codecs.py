"""Number formats of the cache: fp16, OCP fp8-e4m3 and symmetric int8, and the per-block write
rule of the two 8-bit formats.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The pages store the cache in fp16 ("KV Cache Mechanism Explained", section 3.1; "KV Cache and
PagedAttention", section 1.1 and section 5.2) and mention compressing it to fp8 e4m3 with a
scaling factor ("KV Cache Mechanism Explained", section 8, item 3 -- mixed-precision cache; the
snippet there casts to torch.float8_e4m3fn and derives a scale from abs().max()). The printed
snippet is garbled (it takes the max after the cast and divides by the int8 limit 127), so the
rule below is the reading taken for a per-block fp32 scale:

  * e4m3 here is the OCP "fn" variant: 1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent 0
    is subnormal; S.1111.111 is NaN; there is no infinity; the largest finite magnitude is 448.
  * enc(y): round y to the nearest finite e4m3 value, ties to the even code, magnitudes beyond
    448 saturate to 448, the sign bit is kept (so -0 and small negatives give 0x80).
  * A block holds one fp32 scale for K (and one for V) covering every head of the block. Tokens
    are written one at a time in order. Writing in-block slot 0 starts a fresh block (scale 0).
    For a new token x (all heads): s_new = fp32(max|x| / 448); if s_new > scale, the codes
    already in slots [0, off) are re-quantised as enc(fp32(fp32(dec(c) * old) / s_new)) and the
    scale becomes s_new; then the token is stored as enc(fp32(x / scale)). While the scale is 0
    (every value written so far is +-0) a value is stored as a signed zero code.
  * The stored value of a code c in a block with scale s is dec(c) * s.

The int8 cache ("KV Cache Mechanism Explained", section 8, item 3 names FP8/INT8 for the
history tokens with a scaling factor max|x| / 127; "KV Cache and PagedAttention", section 7.2,
8-bit quantisation of blocks) follows the same rule with the int8 limit: codes are two's-
complement int8 in [-127, 127] (-128 is never written), enc(y) = y rounded to the nearest
integer, ties to even, saturated to +-127 (NaN -> 0); s_new = fp32(max|x| / 127); dec(c) = c.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E4M3_NAN = 0x7F


def f16_round(x) -> np.ndarray:
    """Round to IEEE binary16, nearest even (NumPy's conversion)."""
    return np.asarray(x, dtype=np.float64).astype(np.float16)


def e4m3_decode_table() -> np.ndarray:
    """float64 value of every one of the 256 e4m3 codes, from the OCP definition."""
    out = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            out[code] = np.nan
        elif e == 0:
            out[code] = sign * (m / 8.0) * 2.0 ** -6
        else:
            out[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return out


_DEC = e4m3_decode_table()
# magnitudes of the finite non-negative codes 0x00 .. 0x7E, increasing with the code
_MAGS = _DEC[:0x7F].copy()


def e4m3_decode(codes) -> np.ndarray:
    return _DEC[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(y) -> np.ndarray:
    """Nearest finite e4m3 code to each value of y (ties to the even code, saturating at 448,
    sign bit kept, NaN -> 0x7F with the sign). The magnitudes of the finite codes increase with
    the code, so the two candidates for |y| are the first magnitude not below it (binary search
    in that table) and the one before; the nearer wins, and of two equally near the even code."""
    y = np.asarray(y, dtype=np.float64)
    nan = np.isnan(y)
    a = np.minimum(np.where(nan, 0.0, np.abs(y)), E4M3_MAX)   # beyond 448 (and inf) -> 448
    hi = np.searchsorted(_MAGS, a, side="left")                # a <= 448 = _MAGS[-1]
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _MAGS[lo]
    d_hi = _MAGS[hi] - a
    pick = np.where(d_lo < d_hi, lo, np.where(d_hi < d_lo, hi, np.where(lo % 2 == 0, lo, hi)))
    code = np.where(nan, E4M3_NAN, pick).astype(np.uint8)
    return (code | np.where(np.signbit(y), np.uint8(0x80), np.uint8(0))).astype(np.uint8)


def _enc_scaled(y32: np.ndarray, s: np.float32) -> np.ndarray:
    """Codes of fp32 values y32 under fp32 scale s (s == 0 stores signed zeros)."""
    if s == 0:
        return np.where(np.signbit(y32), np.uint8(0x80), np.uint8(0)).astype(np.uint8)
    q = (y32 / np.float32(s)).astype(np.float32)   # IEEE binary32 division, nearest even
    return e4m3_encode(q)


def fp8_write_token(codes: np.ndarray, scale, off: int, x) -> np.float32:
    """Write one token into an fp8 block, per the rule in the module docstring.

    codes: uint8 [H, block_size, D] of one physical block (modified in place);
    scale: the block's current fp32 scale; off: in-block slot of the token;
    x: the token's values, [H, D], exactly representable in fp32.
    Returns the block's new fp32 scale.
    """
    x32 = np.asarray(x, dtype=np.float32)
    s = np.float32(0.0) if off == 0 else np.float32(scale)
    amax = np.float32(np.max(np.abs(x32))) if x32.size else np.float32(0.0)
    s_new = np.float32(amax / np.float32(E4M3_MAX))
    if s_new > s:
        if off > 0:
            old = np.float32(s)
            y = (e4m3_decode(codes[:, :off, :]).astype(np.float32) * old).astype(np.float32)
            codes[:, :off, :] = _enc_scaled(y, s_new)
        s = s_new
    codes[:, off, :] = _enc_scaled(x32, s)
    return np.float32(s)


# ---- int8 --------------------------------------------------------------------------------
I8_MAX = 127.0


def i8_decode(codes) -> np.ndarray:
    return np.asarray(codes, dtype=np.int8).astype(np.float64)


def i8_encode(y) -> np.ndarray:
    """Nearest integer to each value of y (ties to the even integer), saturated to +-127; NaN
    gives 0. Written out from the definition: take floor, compare the remainder with 1/2."""
    y = np.asarray(y, dtype=np.float64)
    nan = np.isnan(y)
    a = np.clip(np.where(nan, 0.0, y), -I8_MAX, I8_MAX)
    f = np.floor(a)
    r = a - f
    up = (r > 0.5) | ((r == 0.5) & (np.mod(f, 2.0) == 1.0))
    return (f + up).astype(np.int8)


def _i8_enc_scaled(y32: np.ndarray, s: np.float32) -> np.ndarray:
    if s == 0:
        return np.zeros(y32.shape, dtype=np.int8)
    with np.errstate(invalid="ignore"):   # a NaN or infinite scale is a defined case (NaN codes)
        return i8_encode((y32 / np.float32(s)).astype(np.float32))


def i8_write_token(codes: np.ndarray, scale, off: int, x) -> np.float32:
    """Write one token into an int8 block: the fp8 rule with the int8 limit 127.

    codes: int8 [H, block_size, D] of one physical block (modified in place); scale: the block's
    current fp32 scale; off: in-block slot; x: [H, D] values exact in fp32. Returns the new
    scale."""
    x32 = np.asarray(x, dtype=np.float32)
    s = np.float32(0.0) if off == 0 else np.float32(scale)
    amax = np.float32(np.max(np.abs(x32))) if x32.size else np.float32(0.0)
    s_new = np.float32(amax / np.float32(I8_MAX))
    if s_new > s:
        if off > 0:
            old = np.float32(s)
            y = (i8_decode(codes[:, :off, :]).astype(np.float32) * old).astype(np.float32)
            codes[:, :off, :] = _i8_enc_scaled(y, s_new)
        s = s_new
    codes[:, off, :] = _i8_enc_scaled(x32, s)
    return np.float32(s)


# ---- whole-block compression ----------------------------------------------------------------
# The pages compress the cached history to 8 bits once it grows past a threshold ("KV Cache
# Mechanism Explained", section 6.1, item 1: dynamic cache compression, fp8 quantisation) and
# compress inactive blocks with 8-bit quantisation ("KV Cache and PagedAttention", section 7.2,
# item 1). Reading taken: a block of a 16-bit cache is re-encoded in one shot into a block of an
# 8-bit cache with the same per-block scale convention as the write rule above: over the block's
# first n_valid slots of every head, s = fp32(max|x| / limit), each of those values is stored as
# enc(fp32(x / s)) (a signed zero code while s = 0), and the slots past n_valid hold code 0 and
# take no part in the scale (their source values are never read).

def compress_block(x, n_valid: int, fmt: str):
    """One-shot 8-bit encoding of one block.

    x: [H, block_size, D] source values, exact in fp32 (slots >= n_valid are ignored and may
    hold anything, NaN included); n_valid: slots 0 .. n_valid-1 hold positions; fmt: "e4m3" or
    "i8". Returns (codes [H, block_size, D] as uint8 for e4m3 / int8 for i8, fp32 scale)."""
    x = np.asarray(x)
    H, bs, D = x.shape
    if not 0 <= n_valid <= bs:
        raise ValueError("n_valid")
    limit = np.float32(E4M3_MAX if fmt == "e4m3" else I8_MAX)
    codes = np.zeros((H, bs, D), dtype=np.uint8 if fmt == "e4m3" else np.int8)
    if n_valid == 0:
        return codes, np.float32(0.0)
    xv = x[:, :n_valid, :].astype(np.float32)
    amax = np.float32(np.max(np.abs(xv)))
    s = np.float32(amax / limit)
    codes[:, :n_valid, :] = _enc_scaled(xv, s) if fmt == "e4m3" else _i8_enc_scaled(xv, s)
    return codes, s
