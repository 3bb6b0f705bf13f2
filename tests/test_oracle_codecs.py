"""Pins for oracle.codecs (CPU only): fp16 and OCP e4m3 against their definitions and against
torch's conversion routines, and the per-block fp8 write rule against its stated properties."""
import numpy as np
import pytest
import torch

from oracle.codecs import (E4M3_MAX, e4m3_decode, e4m3_decode_table, e4m3_encode, f16_round,
                           fp8_write_token)


def test_e4m3_decode_spot_values():
    t = e4m3_decode_table()
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert t[0x38] == 1.0
    assert t[0x08] == 2.0 ** -6          # smallest normal
    assert t[0x01] == 2.0 ** -9          # smallest subnormal
    assert t[0x07] == 7 * 2.0 ** -9
    assert t[0x77] == 240.0
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert t[0x00] == 0.0 and np.signbit(t[0x80])
    fin = t[:0x7F]
    assert np.all(np.diff(fin) > 0)
    assert np.count_nonzero(~np.isnan(t)) == 254


def test_e4m3_decode_matches_torch_all_codes():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = e4m3_decode_table()
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()


def test_e4m3_encode_matches_torch_on_every_fp16_in_range():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    h = h[np.isfinite(h)]
    h = h[np.abs(h.astype(np.float64)) < 464.0]    # torch does not saturate beyond this
    ours = e4m3_encode(h.astype(np.float64))
    ref = torch.from_numpy(h.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(ours, ref)


def test_e4m3_encode_saturates_and_keeps_sign():
    x = np.array([448.0, 463.99, 464.0, 500.0, 1e6, np.inf, -1e6, -np.inf])
    np.testing.assert_array_equal(e4m3_encode(x),
                                  [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE])
    assert e4m3_encode(np.array([np.nan]))[0] & 0x7F == 0x7F
    np.testing.assert_array_equal(e4m3_encode(np.array([-0.0, -1e-9, 0.0, 1e-9])),
                                  [0x80, 0x80, 0x00, 0x00])


def test_e4m3_encode_is_nearest_with_even_ties():
    rng = np.random.default_rng(3)
    y = rng.uniform(-460, 460, 20000) * np.exp2(rng.integers(-14, 1, 20000))
    c = e4m3_encode(y)
    err = np.abs(e4m3_decode(c) - y)
    table = e4m3_decode_table()[:0x7F]
    best = np.abs(np.abs(y)[:, None] - table[None, :]).min(axis=1)
    np.testing.assert_array_equal(err, best)
    # exact midpoints: 1 + 1/16 lies between 1.0 (0x38) and 1.125 (0x39) -> even code 0x38
    assert e4m3_encode(np.array([1.0625]))[0] == 0x38
    assert e4m3_encode(np.array([1.1875]))[0] == 0x3A   # between 0x39 and 0x3A -> 0x3A
    assert e4m3_encode(np.array([2.0 ** -10]))[0] == 0x00   # half of the smallest subnormal
    assert e4m3_encode(np.array([3 * 2.0 ** -10]))[0] == 0x02


def test_f16_round_all_codes_roundtrip_and_ties():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    fin = np.isfinite(h)
    back = f16_round(h[fin].astype(np.float64))
    np.testing.assert_array_equal(back.view(np.uint16), h[fin].view(np.uint16))
    assert f16_round(1 + 2.0 ** -11) == 1.0
    assert f16_round(1 + 3 * 2.0 ** -11) == 1 + 2.0 ** -9


def _block(H=3, D=8):
    return np.zeros((H, 16, D), dtype=np.uint8)


def test_fp8_first_token_scale_and_extreme_code():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((3, 8)).astype(np.float32)
    codes = _block()
    s = fp8_write_token(codes, 0.0, 0, x)
    amax = np.float32(np.abs(x).max())
    assert s == np.float32(amax / np.float32(448.0))
    i = np.unravel_index(np.abs(x).argmax(), x.shape)
    assert codes[i[0], 0, i[1]] & 0x7F == 0x7E
    # every value within half an e4m3 step (relative 2^-4 for normals) of the input
    vals = e4m3_decode(codes[:, 0, :]) * np.float64(s)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * s) * (1 + 1e-6)
    assert np.all(np.abs(vals - x) <= bound)


def test_fp8_single_token_codes_match_torch_quantiser():
    rng = np.random.default_rng(12)
    x = (rng.standard_normal((4, 16)) * 3).astype(np.float16).astype(np.float32)
    codes = np.zeros((4, 16, 16), dtype=np.uint8)
    s = fp8_write_token(codes, 0.0, 0, x)
    q = torch.from_numpy(x) / torch.tensor(s, dtype=torch.float32)
    ref = q.clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(codes[:, 0, :], ref)


def test_fp8_smaller_token_leaves_earlier_codes_untouched():
    rng = np.random.default_rng(13)
    codes = _block()
    x0 = rng.standard_normal((3, 8)).astype(np.float32) * 4
    s0 = fp8_write_token(codes, 0.0, 0, x0)
    before = codes[:, 0, :].copy()
    x1 = x0 * np.float32(0.25)
    s1 = fp8_write_token(codes, s0, 1, x1)
    assert s1 == s0
    np.testing.assert_array_equal(codes[:, 0, :], before)


def test_fp8_growing_scale_requantises_earlier_tokens():
    rng = np.random.default_rng(14)
    codes = _block()
    x0 = rng.standard_normal((3, 8)).astype(np.float32)
    s0 = fp8_write_token(codes, 0.0, 0, x0)
    c0 = codes[:, 0, :].copy()
    x1 = rng.standard_normal((3, 8)).astype(np.float32) * 10
    s1 = fp8_write_token(codes, s0, 1, x1)
    assert s1 == np.float32(np.float32(np.abs(x1).max()) / np.float32(448))
    assert s1 > s0
    # the first token stays within one step at the old scale plus one at the new scale
    v0 = e4m3_decode(codes[:, 0, :]) * np.float64(s1)
    bound = (np.maximum(np.abs(x0) * 2.0 ** -4, 2.0 ** -10 * s0)
             + np.maximum(np.abs(x0) * 1.07 * 2.0 ** -4, 2.0 ** -10 * s1)) * (1 + 1e-6)
    assert np.all(np.abs(v0 - x0) <= bound)
    # the earlier token is requantised from its stored codes (dequantise at the old scale, then
    # quantise at the new one); torch's fp8 conversion does the rounding here
    deq = torch.from_numpy(c0).view(torch.float8_e4m3fn).to(torch.float32) * float(s0)
    ref = (deq / float(s1)).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(codes[:, 0, :], ref)


def test_fp8_slot_zero_restarts_block_and_zero_tokens():
    codes = _block()
    big = np.full((3, 8), 100.0, dtype=np.float32)
    s = fp8_write_token(codes, 0.0, 0, big)
    # a later write at slot 0 ignores the stale scale
    small = np.full((3, 8), 0.5, dtype=np.float32)
    s2 = fp8_write_token(codes, s, 0, small)
    assert s2 == np.float32(np.float32(0.5) / np.float32(448))
    # an all-zero first token keeps scale 0 and signed-zero codes; a later token sets the scale
    codes = _block()
    z = np.zeros((3, 8), dtype=np.float32)
    z[0, 0] = -0.0
    s = fp8_write_token(codes, 0.0, 0, z)
    assert s == 0.0 and np.all((codes[:, 0, :] & 0x7F) == 0)
    s = fp8_write_token(codes, s, 1, small)
    assert s > 0 and np.all((codes[:, 0, :] & 0x7F) == 0)
    assert np.all(codes[:, 1, :] == 0x7E)


@pytest.mark.parametrize("seed", [0, 1])
def test_fp8_token_sequential_error_vs_unquantised(seed):
    """A 16-token block of N(0,1) fp16 data stays within the fp8 tolerance band of 3e-2 relative
    to typical magnitudes once all requantisations are done."""
    rng = np.random.default_rng(seed)
    H, D = 4, 32
    xs = rng.standard_normal((16, H, D)).astype(np.float16).astype(np.float32)
    codes = np.zeros((H, 16, D), dtype=np.uint8)
    s = 0.0
    for t in range(16):
        s = fp8_write_token(codes, s, t, xs[t])
    vals = e4m3_decode(codes) * np.float64(s)           # [H, 16, D]
    err = np.abs(vals - xs.transpose(1, 0, 2))
    assert err.max() < 0.5 and err.mean() < 0.05
    # the scale is the block maximum over all written tokens / 448
    assert s == np.float32(np.float32(np.abs(xs).max()) / np.float32(448))


# ---- int8 ----------------------------------------------------------------------------------
from oracle.codecs import I8_MAX, i8_decode, i8_encode, i8_write_token  # noqa: E402


def test_i8_encode_matches_numpy_rint_and_saturates():
    """Nearest integer, ties to even, is what NumPy's rint does (a library routine); values are
    checked on a fine grid with every half-integer in range, plus saturation and NaN."""
    y = np.concatenate([np.arange(-140.0, 140.0, 0.25), np.arange(-130.5, 131.0, 1.0),
                        np.random.default_rng(3).standard_normal(2000) * 60])
    want = np.clip(np.rint(y), -127, 127).astype(np.int8)
    np.testing.assert_array_equal(i8_encode(y), want)
    assert i8_encode(np.array([0.5, 1.5, 2.5, -0.5, -1.5, -2.5])).tolist() == [0, 2, 2, 0, -2, -2]
    assert i8_encode(np.array([127.5, 1e9, np.inf, -127.5, -np.inf, np.nan])).tolist() == \
        [127, 127, 127, -127, -127, 0]
    np.testing.assert_array_equal(i8_decode(np.arange(-128, 128, dtype=np.int8)),
                                  np.arange(-128.0, 128.0))


def test_i8_first_token_scale_extreme_code_and_error_bound():
    rng = np.random.default_rng(21)
    x = rng.standard_normal((3, 8)).astype(np.float32)
    codes = np.zeros((3, 16, 8), dtype=np.int8)
    s = i8_write_token(codes, 0.0, 0, x)
    assert s == np.float32(np.float32(np.abs(x).max()) / np.float32(I8_MAX))
    i = np.unravel_index(np.abs(x).argmax(), x.shape)
    assert abs(int(codes[i[0], 0, i[1]])) == 127
    vals = i8_decode(codes[:, 0, :]) * np.float64(s)
    assert np.all(np.abs(vals - x) <= 0.5 * s * (1 + 1e-6))
    # the quantiser is round(x / s) with torch's rounding (a library routine), ties to even
    q = torch.round(torch.from_numpy(x) / torch.tensor(s, dtype=torch.float32))
    np.testing.assert_array_equal(codes[:, 0, :], q.clamp(-127, 127).to(torch.int8).numpy())


def test_i8_growing_scale_requantises_and_slot_zero_restarts():
    rng = np.random.default_rng(22)
    codes = np.zeros((2, 16, 8), dtype=np.int8)
    x0 = rng.standard_normal((2, 8)).astype(np.float32)
    s0 = i8_write_token(codes, 0.0, 0, x0)
    c0 = codes[:, 0, :].copy()
    s_same = i8_write_token(codes, s0, 1, x0 * np.float32(0.5))      # smaller: untouched
    assert s_same == s0
    np.testing.assert_array_equal(codes[:, 0, :], c0)
    x2 = rng.standard_normal((2, 8)).astype(np.float32) * 9
    s2 = i8_write_token(codes, s0, 2, x2)
    assert s2 == np.float32(np.float32(np.abs(x2).max()) / np.float32(127)) and s2 > s0
    deq = torch.from_numpy(c0).to(torch.float32) * float(s0)
    ref = torch.round(deq / float(s2)).clamp(-127, 127).to(torch.int8).numpy()
    np.testing.assert_array_equal(codes[:, 0, :], ref)
    # slot 0 ignores a stale scale; an all-zero first token keeps scale 0 and zero codes
    s3 = i8_write_token(codes, s2, 0, x0)
    assert s3 == s0
    z = np.zeros((2, 16, 8), dtype=np.int8)
    assert i8_write_token(z, 0.0, 0, np.zeros((2, 8), np.float32)) == 0.0 and not z.any()


def test_i8_token_sequential_error_vs_unquantised():
    rng = np.random.default_rng(23)
    H, D = 4, 32
    xs = rng.standard_normal((16, H, D)).astype(np.float16).astype(np.float32)
    codes = np.zeros((H, 16, D), dtype=np.int8)
    s = 0.0
    scales = []
    for t in range(16):
        s = i8_write_token(codes, s, t, xs[t])
        scales.append(float(s))
    vals = i8_decode(codes) * np.float64(s)
    err = np.abs(vals - xs.transpose(1, 0, 2))          # [H, 16, D]
    # token t was rounded once at its own scale and once more at every larger scale that came
    # after it: each rounding moves it by at most half a step of that scale
    for t in range(16):
        bound = 0.5 * sum(sorted(set(scales[t:])))
        assert err[:, t, :].max() <= bound * (1 + 1e-6), t
    assert s == np.float32(np.float32(np.abs(xs).max()) / np.float32(127))


# ---- whole-block compression ---------------------------------------------------------------
from oracle.codecs import E4M3_MAX, compress_block, e4m3_decode  # noqa: E402


@pytest.mark.parametrize("fmt", ["e4m3", "i8"])
def test_compress_block_scale_extreme_code_and_error_bound(fmt):
    """The scale is max|x| / limit over the valid slots of every head; the element of largest
    magnitude gets the extreme code (+-limit exactly); every stored value is within the
    format's half step of the source (int8: s/2; e4m3: 2^-4 relative, or 2^-10 s absolute
    in the subnormal range)."""
    g = np.random.default_rng(31)
    x = g.standard_normal((3, 16, 32)).astype(np.float16).astype(np.float32)
    n = 11
    x[:, n:, :] = np.nan                               # past the valid slots: never read
    codes, s = compress_block(x, n, fmt)
    lim = np.float32(E4M3_MAX if fmt == "e4m3" else I8_MAX)
    xv = x[:, :n, :]
    assert s == np.float32(np.float32(np.abs(xv).max()) / lim)
    dec = e4m3_decode(codes) if fmt == "e4m3" else i8_decode(codes)
    vals = dec[:, :n, :] * np.float64(s)
    k = np.unravel_index(np.argmax(np.abs(xv)), xv.shape)
    assert abs(dec[:, :n, :][k]) == float(lim)
    err = np.abs(vals - xv.astype(np.float64))
    if fmt == "i8":
        assert err.max() <= 0.5 * float(s) * (1 + 1e-6)
    else:
        bound = np.maximum(np.abs(xv) * 2.0 ** -4, 2.0 ** -10 * float(s))
        assert np.all(err <= bound * (1 + 1e-6))
    assert not codes[:, n:, :].any()                   # past n_valid: code 0


@pytest.mark.parametrize("fmt", ["e4m3", "i8"])
def test_compress_block_degenerate_cases(fmt):
    z = np.zeros((2, 16, 8), np.float32)
    codes, s = compress_block(z, 16, fmt)
    assert s == 0.0 and not codes.any()
    codes, s = compress_block(np.full((2, 16, 8), np.nan, np.float32), 0, fmt)
    assert s == 0.0 and not codes.any()
    # negative zeros: e4m3 keeps the sign code, int8 has none
    neg = np.full((1, 16, 4), -0.0, np.float32)
    codes, s = compress_block(neg, 16, fmt)
    assert s == 0.0
    assert (codes == (0x80 if fmt == "e4m3" else 0)).all()
    with pytest.raises(ValueError):
        compress_block(z, 17, fmt)


@pytest.mark.parametrize("fmt", ["e4m3", "i8"])
def test_compress_block_equals_writer_when_the_first_token_holds_the_maximum(fmt):
    """When the block's largest magnitude arrives with its first token, the running-scale
    writer never requantises, so writing the tokens one by one gives the one-shot encoding."""
    g = np.random.default_rng(32)
    x = g.standard_normal((2, 16, 16)).astype(np.float32)
    x[:, 0, :] *= 8.0
    x[0, 0, 0] = 40.0                                  # the maximum, in slot 0
    n = 13
    write = fp8_write_token if fmt == "e4m3" else i8_write_token
    codes = np.zeros(x.shape, np.uint8 if fmt == "e4m3" else np.int8)
    s = 0.0
    for t in range(n):
        s = write(codes, s, t, x[:, t, :])
    c1, s1 = compress_block(x, n, fmt)
    assert s1 == s
    np.testing.assert_array_equal(c1, codes)


def test_compress_block_ties_go_to_even_codes():
    """At scale 1 (block maximum equal to the limit) a value half-way between two codes takes
    the even one: int8 k + 1/2 -> the even integer; e4m3 midpoints -> the code with an even
    last mantissa bit. A NaN among the valid values makes the scale NaN (and int8 codes 0)."""
    k = np.arange(-127, 127, dtype=np.float64)
    x = np.zeros((1, 16, 256), np.float32)
    x[0, 0, :254] = k + 0.5
    x[0, 1, 0] = 127.0
    codes, s = compress_block(x, 16, "i8")
    assert s == 1.0
    want = np.where(np.mod(k, 2) == 0, k, k + 1)
    np.testing.assert_array_equal(codes[0, 0, :254].astype(np.int64), want.astype(np.int64))
    # e4m3: 1.0 (0x38) and 1.125 (0x39) -> midpoint 1.0625 goes to 0x38; 1.1875 to 0x3A (1.25)
    y = np.zeros((1, 16, 4), np.float32)
    y[0, 0, :3] = [1.0625, 1.1875, -1.0625]
    y[0, 1, 0] = 448.0
    c8, s8 = compress_block(y, 16, "e4m3")
    assert s8 == 1.0
    assert list(c8[0, 0, :3]) == [0x38, 0x3A, 0xB8]
    nan = x.copy()
    nan[0, 2, 3] = np.nan
    c, s = compress_block(nan, 16, "i8")
    assert np.isnan(s) and not c.any()
