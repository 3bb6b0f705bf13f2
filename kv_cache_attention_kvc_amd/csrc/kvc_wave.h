// Wave-level device helpers shared by the HIP translation units of libkvc (not part of the
// ABI): cross-lane exchanges, streaming loads, fp16 vector types for the matrix cores, exact
// e4m3-to-fp16 and int8-to-fp16 conversions, and the LDS ordering point between lanes of one
// wavefront.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace kvc {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kFloor = -3.0e38f;  // initial running max (finite, so m - m' is never NaN)

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// The value of x in this lane and in a partner lane OFF lanes away, as an unordered pair
// {a, b} (so a symmetric combination of a and b is the same in both lanes). OFF = 32 and 16 use
// the gfx950 lane-swap instructions (halves of the wave, neighbouring rows of 16); OFF = 8 and 4
// rotate within a row of 16 (row_ror), which pairs lane i with lane i+OFF mod 16.
template <int OFF>
__device__ __forceinline__ void lane_pair(float x, float &a, float &b) {
  const uint32_t u = __float_as_uint(x);
  if constexpr (OFF == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
  } else if constexpr (OFF == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
  } else {
    static_assert(OFF == 8 || OFF == 4, "lane distance 4, 8, 16 or 32");
    a = x;
    b = dpp<0x120 + OFF>(x);  // row_ror:OFF
  }
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 16-byte streaming load (non-temporal hint).
__device__ __forceinline__ uint4 load_stream(const char *p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Ordering point for LDS traffic between the lanes of one wavefront: the compiler keeps LDS
// accesses on their side of it, and the LDS executes one wavefront's accesses in issue order.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Bit view of 16 loaded bytes as 8 fp16 values.
__device__ __forceinline__ f16x8 as_f16x8(const uint4 &u) { return __builtin_bit_cast(f16x8, u); }

// 8 e4m3 codes (two words, lowest byte first) as fp16, exactly: every e4m3 value is an fp16 value
// (gfx950 v_cvt_scalef32_pk_f16_fp8 with scale 1).
__device__ __forceinline__ f16x8 fp8x8_to_f16(uint32_t w0, uint32_t w1) {
#define KVC_CVT8(w, hi) \
  __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(static_cast<int>(w), 1.0f, hi))
  return __builtin_bit_cast(f16x8, make_uint4(KVC_CVT8(w0, false), KVC_CVT8(w0, true),
                                              KVC_CVT8(w1, false), KVC_CVT8(w1, true)));
#undef KVC_CVT8
}

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// 4 int8 codes (one word, lowest byte first) as two fp16 pairs, exactly. Each byte b is biased
// to u = b ^ 0x80 = b + 128 and placed under the fp16 exponent of 1024 (bits 0x6400 | u, the
// value 1024 + u, exact since fp16 steps by 1 in [1024, 2048)); subtracting 1152 leaves b.
// v_perm_b32 picks bytes of {S0, S1} (selector 0-3: S1's bytes, 4-7: S0's).
__device__ __forceinline__ void i8x4_to_f16(uint32_t w, f16x2 &lo, f16x2 &hi) {
  const uint32_t x = w ^ 0x80808080u;
  const f16x2 bias = {static_cast<_Float16>(1152.0f), static_cast<_Float16>(1152.0f)};
  lo = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(0x64646464u, x, 0x04010400u)) - bias;
  hi = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(0x64646464u, x, 0x04030402u)) - bias;
}

// 8 int8 codes (two words) as fp16, exactly.
__device__ __forceinline__ f16x8 i8x8_to_f16(uint32_t w0, uint32_t w1) {
  f16x2 a, b, c, d;
  i8x4_to_f16(w0, a, b);
  i8x4_to_f16(w1, c, d);
  return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

}  // namespace kvc
