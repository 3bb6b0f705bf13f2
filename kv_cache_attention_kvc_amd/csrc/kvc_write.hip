// Cache writes for gfx950: contiguous append, paged scatter, 8-bit (fp8-e4m3 or int8) per-block
// quantised writes, and copy-on-write block copies.
//
// The new token's K/V are stored before attention reads the cache ("LLM Inference Acceleration
// -- KV Cache", section 3.1). Paged writes go to slot = block*16 + offset chosen by the host pool
// ("KV Cache and PagedAttention", sections 3.1 and 3.3). 8-bit pools hold OCP e4m3 or int8 codes
// with one fp32 scale per block for K and one for V ("KV Cache Mechanism Explained", section 8,
// item 3: FP8/INT8 history with a scaling factor; "KV Cache and PagedAttention", section 7.2).
#include "kvc_internal.h"
#include "kvc_wave.h"

namespace kvc {

constexpr int kThreads = 256;

// ---- plain copies ------------------------------------------------------------------------
// One thread per 16-byte chunk of every new (token, head) row, for K and for V: all loads of a
// call are in flight at once.
__global__ void __launch_bounds__(kThreads)
append_contig_kernel(char *kc, char *vc, const char *kn, const char *vn, const int32_t *pos,
                     int32_t B, int32_t H, int32_t S_max, int32_t n_tok, int32_t row_bytes) {
  const int32_t cpr = row_bytes / 16;  // 16-byte chunks per row
  const int64_t x = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (x >= static_cast<int64_t>(B) * n_tok * H * cpr) return;
  const int32_t ch = static_cast<int32_t>(x % cpr);
  const int64_t row = x / cpr;  // (b, t, h) in k_new order
  const int32_t h = static_cast<int32_t>(row % H);
  const int64_t bt = row / H;
  const int32_t t = static_cast<int32_t>(bt % n_tok);
  const int32_t b = static_cast<int32_t>(bt / n_tok);
  const int64_t p = static_cast<int64_t>(pos[b]) + t;
  const uint4 k = *reinterpret_cast<const uint4 *>(kn + row * row_bytes + ch * 16);
  const uint4 v = *reinterpret_cast<const uint4 *>(vn + row * row_bytes + ch * 16);
  if (p < 0 || p >= S_max) return;
  const int64_t dst = ((static_cast<int64_t>(b) * H + h) * S_max + p) * row_bytes + ch * 16;
  *reinterpret_cast<uint4 *>(kc + dst) = k;
  *reinterpret_cast<uint4 *>(vc + dst) = v;
}

// pool[(blk*H + h)*16 + off][:] = new[i][h][:], one thread per 16-byte chunk.
__global__ void __launch_bounds__(kThreads)
write_paged_kernel(char *kp, char *vp, const char *kn, const char *vn, const int64_t *slots,
                   int32_t n_tok, int32_t H, int32_t num_blocks, int32_t row_bytes) {
  const int32_t cpr = row_bytes / 16;
  const int64_t x = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (x >= static_cast<int64_t>(n_tok) * H * cpr) return;
  const int32_t ch = static_cast<int32_t>(x % cpr);
  const int64_t row = x / cpr;  // (i, h) in k_new order
  const int32_t h = static_cast<int32_t>(row % H);
  const int64_t i = row / H;
  const int64_t slot = slots[i];
  const uint4 k = *reinterpret_cast<const uint4 *>(kn + row * row_bytes + ch * 16);
  const uint4 v = *reinterpret_cast<const uint4 *>(vn + row * row_bytes + ch * 16);
  if (slot < 0 || slot >= static_cast<int64_t>(num_blocks) * kBlock) return;
  const int64_t blk = slot / kBlock;
  const int32_t off = static_cast<int32_t>(slot % kBlock);
  const int64_t dst = ((blk * H + h) * kBlock + off) * row_bytes + ch * 16;
  *reinterpret_cast<uint4 *>(kp + dst) = k;
  *reinterpret_cast<uint4 *>(vp + dst) = v;
}

// Copy-on-write copies: workgroup (pair i, slice z) copies 16-byte pieces z*kCopyPieces ..
// + kCopyPieces - 1 of pair i's block (all heads) of K and of V; the first slice also copies the
// 8-bit scales. Every thread issues all its loads before its first store, so a workgroup makes
// one memory round trip, and a pair's block is spread over many workgroups.
constexpr int kCopyUnroll = 4;
constexpr int kCopyPieces = kThreads * kCopyUnroll;

__global__ void __launch_bounds__(kThreads)
copy_blocks_kernel(char *kp, char *vp, float *ks, float *vs, const int32_t *src,
                   const int32_t *dst, int32_t num_blocks, int64_t block_bytes, int32_t slices) {
  const int32_t pair = blockIdx.x / slices;
  const int32_t z = blockIdx.x % slices;
  const int32_t s = src[pair];
  const int32_t d = dst[pair];
  if (static_cast<uint32_t>(s) >= static_cast<uint32_t>(num_blocks) ||
      static_cast<uint32_t>(d) >= static_cast<uint32_t>(num_blocks) || s == d)
    return;
  const int64_t pieces = block_bytes / 16;
  const int64_t so = static_cast<int64_t>(s) * block_bytes;
  const int64_t dof = static_cast<int64_t>(d) * block_bytes;
  uint4 kx[kCopyUnroll], vx[kCopyUnroll];
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const int64_t c = static_cast<int64_t>(z) * kCopyPieces + u * kThreads + threadIdx.x;
    if (c < pieces) {
      kx[u] = *reinterpret_cast<const uint4 *>(kp + so + c * 16);
      vx[u] = *reinterpret_cast<const uint4 *>(vp + so + c * 16);
    }
  }
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const int64_t c = static_cast<int64_t>(z) * kCopyPieces + u * kThreads + threadIdx.x;
    if (c < pieces) {
      *reinterpret_cast<uint4 *>(kp + dof + c * 16) = kx[u];
      *reinterpret_cast<uint4 *>(vp + dof + c * 16) = vx[u];
    }
  }
  if (z == 0 && threadIdx.x == 0 && ks) {
    ks[d] = ks[s];
    vs[d] = vs[s];
  }
}

// ---- fp8 e4m3 ----------------------------------------------------------------------------
// Nearest e4m3 code of q (ties to even, saturating to +-448, sign kept, NaN -> 0x7F|sign).
__device__ __forceinline__ uint32_t e4m3_encode(float q) {
  const uint32_t u = __float_as_uint(q);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return sign | 0x7Fu;   // NaN
  if (a >= 0x43E00000u) return sign | 0x7Eu;  // |q| >= 448, infinities included
  if (a < 0x3C800000u) {                      // |q| < 2^-6: subnormal steps of 2^-9
    const float m = __builtin_rintf(__uint_as_float(a) * 512.0f);
    return sign | static_cast<uint32_t>(m);   // 0..8; 8 is the smallest normal code
  }
  const uint32_t e = (a >> 23) - 120u;        // e4m3 exponent field, 1..15
  const uint32_t mant = a & 0x7FFFFFu;
  const uint32_t m3 = mant >> 20;
  const uint32_t rem = mant & 0xFFFFFu;
  uint32_t code = (e << 3) | m3;
  if (rem > 0x80000u || (rem == 0x80000u && (m3 & 1u))) code += 1u;
  return sign | code;
}

// Exact value of a finite e4m3 code.
__device__ __forceinline__ float e4m3_decode(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u;
  const uint32_t m = c & 7u;
  const float mag = e == 0 ? static_cast<float>(m) * 0.001953125f
                           : __uint_as_float(((e + 120u) << 23) | (m << 20));
  return __uint_as_float(__float_as_uint(mag) | ((c & 0x80u) << 24));
}

// int8: nearest integer of q (ties to even, v_rndne), saturated to +-127; NaN -> 0.
__device__ __forceinline__ uint32_t i8_encode(float q) {
  if (!(q == q)) return 0u;
  const float r = __builtin_rintf(fminf(fmaxf(q, -127.0f), 127.0f));
  return static_cast<uint32_t>(static_cast<int32_t>(r)) & 0xFFu;
}

__device__ __forceinline__ float i8_decode(uint32_t c) {
  return static_cast<float>(static_cast<int8_t>(static_cast<uint8_t>(c)));
}

// The two 8-bit formats: code limit, encode (of an fp32 value already divided by the scale),
// exact decode, and the code of a value stored while the scale is 0.
template <int FMT>
struct Q8 {
  static constexpr float kMax = FMT == KVC_E4M3 ? 448.0f : 127.0f;
  static __device__ __forceinline__ uint32_t enc(float q) {
    if constexpr (FMT == KVC_E4M3) return e4m3_encode(q);
    return i8_encode(q);
  }
  static __device__ __forceinline__ float dec(uint32_t c) {
    if constexpr (FMT == KVC_E4M3) return e4m3_decode(c);
    return i8_decode(c);
  }
  static __device__ __forceinline__ uint32_t zero(float x) {
    if constexpr (FMT == KVC_E4M3) return (__float_as_uint(x) >> 24) & 0x80u;  // signed zero
    return 0u;
  }
};

template <int FMT>
__device__ __forceinline__ uint32_t enc_scaled(float x, float s) {
  if (s == 0.f) return Q8<FMT>::zero(x);
  return Q8<FMT>::enc(x / s);
}

__device__ __forceinline__ float block_max(float v, float *red) {
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < kThreads / 64; ++i) r = fmaxf(r, red[i]);
  __syncthreads();
  return r;
}

template <bool SRC_F16>
__device__ __forceinline__ void load4(const void *p, int64_t idx, float *x) {
  if (SRC_F16) {
    const uint2 r = *reinterpret_cast<const uint2 *>(reinterpret_cast<const _Float16 *>(p) + idx);
    x[0] = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(r.x)));
    x[1] = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(r.x >> 16)));
    x[2] = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(r.y)));
    x[3] = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(r.y >> 16)));
  } else {
    const float4 r = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(p) + idx);
    x[0] = r.x;
    x[1] = r.y;
    x[2] = r.z;
    x[3] = r.w;
  }
}

template <int FMT>
__device__ __forceinline__ void requant_rows(uint8_t *pool, int64_t row0, int32_t D, int32_t d,
                                             int32_t off, float old_s, float new_s) {
  for (int t = 0; t < off; ++t) {
    uint32_t *w = reinterpret_cast<uint32_t *>(pool + (row0 + t) * D + d);
    const uint32_t old = *w;
    uint32_t nw = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float y = Q8<FMT>::dec((old >> (8 * u)) & 0xFFu) * old_s;
      nw |= enc_scaled<FMT>(y, new_s) << (8 * u);
    }
    *w = nw;
  }
}

// One workgroup per run of adjacent entries that target the same block; tokens of the run are
// applied in order. Each thread owns the same 4 consecutive elements of every (head, slot) row
// of the block, for all 16 slots, so requantisation only reads bytes the same thread wrote.
// FMT: KVC_E4M3 or KVC_I8.
template <bool SRC_F16, int FMT>
__global__ void __launch_bounds__(kThreads)
write_paged_q8_kernel(uint8_t *kp, uint8_t *vp, float *ks, float *vs, const void *kn,
                       const void *vn, const int64_t *slots, int32_t n_tok, int32_t H, int32_t D,
                       int32_t num_blocks) {
  __shared__ float red[2][kThreads / 64];
  const int32_t i0 = blockIdx.x;
  const int64_t blk = slots[i0] >= 0 ? slots[i0] / kBlock : -1;
  if (i0 > 0) {
    const int64_t prev = slots[i0 - 1];
    if ((prev >= 0 ? prev / kBlock : -1) == blk) return;  // not the start of a run
  }
  if (blk < 0 || blk >= num_blocks) return;
  const int32_t HD = H * D;
  float sk = ks[blk];
  float sv = vs[blk];
  for (int32_t i = i0; i < n_tok; ++i) {
    const int64_t slot = slots[i];
    if (slot < 0 || slot / kBlock != blk) break;
    const int32_t off = static_cast<int32_t>(slot % kBlock);
    if (off == 0) {  // a fresh block: earlier contents and scale are stale
      sk = 0.f;
      sv = 0.f;
    }
    const int64_t base = static_cast<int64_t>(i) * HD;
    float mk = 0.f, mv = 0.f;
    for (int32_t e0 = threadIdx.x * 4; e0 < HD; e0 += 4 * kThreads) {
      float a[4], b[4];
      load4<SRC_F16>(kn, base + e0, a);
      load4<SRC_F16>(vn, base + e0, b);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        mk = fmaxf(mk, fabsf(a[u]));
        mv = fmaxf(mv, fabsf(b[u]));
      }
    }
    mk = block_max(mk, red[0]);
    mv = block_max(mv, red[1]);
    const float nk = mk / Q8<FMT>::kMax;
    const float nv = mv / Q8<FMT>::kMax;
    const bool gk = nk > sk;
    const bool gv = nv > sv;
    const float ck = gk ? nk : sk;
    const float cv = gv ? nv : sv;
    for (int32_t e0 = threadIdx.x * 4; e0 < HD; e0 += 4 * kThreads) {
      const int32_t h = e0 / D;
      const int32_t d = e0 % D;
      const int64_t row0 = (blk * H + h) * kBlock;  // slot-0 row of this head in the block
      if (gk && off > 0) requant_rows<FMT>(kp, row0, D, d, off, sk, nk);
      if (gv && off > 0) requant_rows<FMT>(vp, row0, D, d, off, sv, nv);
      float a[4], b[4];
      load4<SRC_F16>(kn, base + e0, a);
      load4<SRC_F16>(vn, base + e0, b);
      uint32_t wk = 0, wv = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        wk |= enc_scaled<FMT>(a[u], ck) << (8 * u);
        wv |= enc_scaled<FMT>(b[u], cv) << (8 * u);
      }
      *reinterpret_cast<uint32_t *>(kp + (row0 + off) * D + d) = wk;
      *reinterpret_cast<uint32_t *>(vp + (row0 + off) * D + d) = wv;
    }
    sk = ck;
    sv = cv;
  }
  if (threadIdx.x == 0) {
    ks[blk] = sk;
    vs[blk] = sv;
  }
}


// Whole-block compression: one workgroup per (source, destination) pair. The first n slots of
// every head of source block src[i] (fp16 or fp32) are re-encoded into destination block dst[i]
// of an 8-bit layer in one shot: the block's K scale (and V scale) is max|x| / limit over those
// values, every value is stored as enc(x / scale), and slots n .. 15 get code 0. Pairs whose
// ids lie outside their pools are skipped. Each thread takes 4 consecutive elements of a row.
template <bool SRC_F16, int FMT>
__global__ void __launch_bounds__(kThreads)
compress_blocks_kernel(const void *sk, const void *sv, uint8_t *dk, uint8_t *dv, float *ks,
                       float *vs, const int32_t *src, const int32_t *dst, const int32_t *nval,
                       int32_t H, int32_t D, int32_t src_blocks, int32_t dst_blocks) {
  __shared__ float red[2][kThreads / 64];
  const int32_t sb = src[blockIdx.x];
  const int32_t db = dst[blockIdx.x];
  if (static_cast<uint32_t>(sb) >= static_cast<uint32_t>(src_blocks) ||
      static_cast<uint32_t>(db) >= static_cast<uint32_t>(dst_blocks))
    return;
  const int32_t n = nval ? min(max(nval[blockIdx.x], 0), kBlock) : kBlock;
  const int32_t per_block = H * kBlock * D;  // elements of one block of K (or V)
  const int64_t s0 = static_cast<int64_t>(sb) * per_block;
  const int64_t d0 = static_cast<int64_t>(db) * per_block;
  float mk = 0.f, mv = 0.f;
  for (int32_t e0 = threadIdx.x * 4; e0 < per_block; e0 += 4 * kThreads) {
    if ((e0 / D) % kBlock >= n) continue;  // slot past the valid ones: never read
    float a[4], b[4];
    load4<SRC_F16>(sk, s0 + e0, a);
    load4<SRC_F16>(sv, s0 + e0, b);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      mk = fmaxf(mk, fabsf(a[u]));
      mv = fmaxf(mv, fabsf(b[u]));
    }
  }
  mk = block_max(mk, red[0]);
  mv = block_max(mv, red[1]);
  const float ck = mk / Q8<FMT>::kMax;
  const float cv = mv / Q8<FMT>::kMax;
  for (int32_t e0 = threadIdx.x * 4; e0 < per_block; e0 += 4 * kThreads) {
    uint32_t wk = 0, wv = 0;
    if ((e0 / D) % kBlock < n) {
      float a[4], b[4];
      load4<SRC_F16>(sk, s0 + e0, a);
      load4<SRC_F16>(sv, s0 + e0, b);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        wk |= enc_scaled<FMT>(a[u], ck) << (8 * u);
        wv |= enc_scaled<FMT>(b[u], cv) << (8 * u);
      }
    }
    *reinterpret_cast<uint32_t *>(dk + d0 + e0) = wk;
    *reinterpret_cast<uint32_t *>(dv + d0 + e0) = wv;
  }
  if (threadIdx.x == 0) {
    ks[db] = ck;
    vs[db] = cv;
  }
}


// Single-read compression of fp16 blocks. A unit is (pair, K or V); its block (H*16*D fp16) is
// held in registers between the block maximum and the encoding, NL 16-byte pieces per thread at
// most, so each source byte is read from memory once. Thread t takes pieces t, t + T, ...; a
// piece is 8 consecutive values of one (head, slot) row. Blocks of up to 8192 pieces run on the
// streaming kernel below (T = 512, NL = 4, 8 or 16, the smallest that covers the block); larger
// ones, up to 16384 pieces, take one 1024-thread workgroup per unit.
//
// Encoding is instruction-bound, not memory-bound, if every value pays an IEEE division, so the
// codes come from v = x * r with r = RN(1/s), rounded once (fused), and each value whose v lies
// close to a rounding boundary of the format is redone with the division. Bound: r is within
// 2^-24 relative of 1/s and the product adds one rounding, so v is within 2^-23 relative of x/s,
// and RN(x/s) within 2^-24 of it; |x/s| <= limit*(1 + 2^-24) since |x| <= max|x| and
// s = RN(max|x| / limit). A boundary further from v than that leaves RN(x/s) on v's side, so
// both round to the same code. The shortcut needs a finite, non-zero s; a block maximum that is
// 0, infinite or NaN gives fixed codes (degenerate_code), with no division at all.
constexpr int kCompMaxPieces = 1024 * 16;   // H*D <= 8192 (e.g. 64 heads of 128)

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Lane-wise unsigned maximum of two pairs of 16-bit fields.
__device__ __forceinline__ uint32_t max_u16x2(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                __builtin_bit_cast(u16x2, b)));
}

// fma(fp16 x, r, c) with one rounding (v_fma_mix_f32; x is widened exactly).
__device__ __forceinline__ float fma_f16_f32(_Float16 x, float r, float c) {
  return __builtin_fmaf(static_cast<float>(x), r, c);
}

// int8: v = RN(x*r + 128) is within 2^-16 + 2^-17 of x/s + 128 (|x/s| <= 127 + 2^-16), and
// RN(x/s) within 2^-18 of x/s; a half-integer further than 2^-14 from v therefore lies on neither
// side, and rint(v) - 128 is the code. The result is the code + 128 as a float (1 .. 255).
__device__ __forceinline__ float i8_biased_code(_Float16 x, float r, float s) {
  const float v = fma_f16_f32(x, r, 128.0f);
  const float t = __builtin_rintf(v);
  if (__builtin_expect(fabsf(v - t) > 0.5f - 0x1p-14f, 0))  // near a tie: exact quotient
    return __builtin_rintf(fminf(fmaxf(static_cast<float>(x) / s, -127.0f), 127.0f)) + 128.0f;
  return t;
}

// e4m3: v = RN(x*r) (sign of zero kept) is within 3 units in the last place (fp32) of RN(x/s).
// In the normal range the code is v's top 3 mantissa bits rounded to nearest even, unless the 20
// bits below lie within 8 units of the half-way pattern; codes below 2^-6 (subnormal steps)
// and zeros take the exact path. No saturation arises: |v| < 464 rounds to at most 448.
__device__ __forceinline__ uint32_t e4m3_code(_Float16 x, float r, float s) {
  const uint32_t u = __float_as_uint(fma_f16_f32(x, r, -0.0f));
  const uint32_t a = u & 0x7FFFFFFFu;
  const uint32_t rem = a & 0xFFFFFu;
  const bool hard = a < 0x3C800000u || (rem - 0x7FFF8u) <= 16u;
  if (__builtin_expect(hard, 0)) return e4m3_encode(static_cast<float>(x) / s);
  // exponent rebias 127 -> 7 and round-to-nearest-even on the 20 dropped bits; the sign moves
  // from bit 11 to bit 7 (bits 7..10 are zero for |v| in [2^-6, 464))
  const uint32_t c = (u + 0x7FFFFu - (120u << 23) + ((u >> 20) & 1u)) >> 20;
  return (c & 0x7Fu) | ((c >> 4) & 0x80u);
}

// Code of x/s for a scale that is 0 (the block holds only zeros), +inf (an infinite value in
// the block) or NaN (a NaN in the block), without the division: x/0 is never formed (zeros keep
// their sign in e4m3); x/inf is a signed zero for finite x and NaN for infinite x; x/NaN is NaN.
// NaN codes are 0 in int8 and 0x7F in e4m3 (the quotient NaN is the positive default NaN).
template <int FMT>
__device__ __forceinline__ uint32_t degenerate_code(_Float16 x, float s) {
  if constexpr (FMT == KVC_I8) {
    return 0u;
  } else {
    const uint32_t b = __builtin_bit_cast(uint16_t, x);
    const uint32_t sign = (b >> 8) & 0x80u;
    const bool x_finite = (b & 0x7C00u) != 0x7C00u;
    if (s == 0.f || (s > 0.f && x_finite)) return sign;
    return 0x7Fu;
  }
}

// Codes of the thread's piece pairs (see compress_f16_regs_kernel), stored 16 bytes a pair; FAST
// takes the reciprocal path (finite, non-zero scale), else every value is divided.
template <int FMT, int NL, int T, bool FAST>
__device__ __forceinline__ void encode_pairs(const uint4 (&x)[NL], uint32_t keep_bits,
                                             int32_t pieces, uint8_t *dp, float sc) {
  const float r = FAST ? 1.0f / sc : 0.f;
#pragma unroll
  for (int i = 0; i < NL / 2; ++i) {
    // the pair index is formed here, not kept from the loads: holding NL/2 offsets across the
    // encoding would take registers the data needs
    int32_t t = threadIdx.x;
    asm volatile("" : "+v"(t));
    const int32_t c = 2 * (t + i * T);
    if (c >= pieces) continue;
    const uint32_t keep = 0u - ((keep_bits >> i) & 1u);
    uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const f16x8 h = as_f16x8(x[2 * i + k]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint32_t &wd = w[2 * k + e / 4];
        if constexpr (!FAST)
          wd |= degenerate_code<FMT>(h[e], sc) << (8 * (e % 4));
        else if constexpr (FMT == KVC_I8)
          wd = __builtin_amdgcn_cvt_pk_u8_f32(i8_biased_code(h[e], r, sc), e % 4, wd);
        else
          wd |= e4m3_code(h[e], r, sc) << (8 * (e % 4));
      }
    }
    if constexpr (FAST && FMT == KVC_I8) {  // biased bytes back to two's complement
#pragma unroll
      for (int j = 0; j < 4; ++j) w[j] ^= 0x80808080u;
    }
    *reinterpret_cast<uint4 *>(dp + static_cast<int64_t>(c) * 8) =
        make_uint4(w[0] & keep, w[1] & keep, w[2] & keep, w[3] & keep);
  }
}

// One (pair, K or V) unit of a compression call: its source pieces, destination codes and scale
// slot, its valid slots, and whether both ids lie in their pools (a unit outside them is skipped;
// its loads read block 0 of the source instead).
struct CompUnit {
  const char *sp;
  uint8_t *dp;
  float *scale;
  int32_t n;
  bool ok;
};

struct CompArgs {
  const char *sk, *sv;
  uint8_t *dk, *dv;
  float *ks, *vs;
  const int32_t *src, *dst, *nval;
  int32_t H, D, src_blocks, dst_blocks;
  int32_t n_units;  // 2 * pairs
};

// Read-only int32 at a wave-uniform address, through the scalar cache: its completion is counted
// apart from the vector loads, so waiting for a unit's ids never waits for block data in flight.
typedef const __attribute__((address_space(4))) int32_t comp_const_i32;
__device__ __forceinline__ int32_t comp_sload(const int32_t *p) {
  return *(comp_const_i32 *)(p);
}

__device__ __forceinline__ CompUnit comp_unit(const CompArgs &a, int32_t u) {
  const int32_t pair = u >> 1;
  const bool is_v = u & 1;
  const int32_t sb = comp_sload(a.src + pair);
  const int32_t db = comp_sload(a.dst + pair);
  CompUnit c;
  c.ok = static_cast<uint32_t>(sb) < static_cast<uint32_t>(a.src_blocks) &&
         static_cast<uint32_t>(db) < static_cast<uint32_t>(a.dst_blocks);
  const int64_t pieces = static_cast<int64_t>(a.H) * kBlock * a.D / 8;
  c.sp = (is_v ? a.sv : a.sk) + (c.ok ? sb : 0) * pieces * 16;
  c.dp = (is_v ? a.dv : a.dk) + (c.ok ? db : 0) * pieces * 8;
  c.scale = (is_v ? a.vs : a.ks) + (c.ok ? db : 0);
  c.n = a.nval ? min(max(comp_sload(a.nval + pair), 0), kBlock) : kBlock;
  return c;
}

// Thread t takes the piece pairs (2u, 2u + 1), u = t + i * T: both pieces lie in one (head, slot)
// row (a row has D/8 >= 8 pieces), and their 16 codes form one 16-byte store. Every load is
// issued before any is used (a load per branch would wait for each in turn); pairs past the block
// read its first pair instead.
template <int NL, int T>
__device__ __forceinline__ void load_pieces(const char *sp, int32_t pieces, uint4 (&x)[NL]) {
#pragma unroll
  for (int i = 0; i < NL / 2; ++i) {
    const int32_t c = 2 * (threadIdx.x + i * T);
    const int64_t off = static_cast<int64_t>(c < pieces ? c : 0) * 16;
    x[2 * i] = *reinterpret_cast<const uint4 *>(sp + off);
    x[2 * i + 1] = *reinterpret_cast<const uint4 *>(sp + off + 16);
  }
}

// The unit's scale and codes from its pieces in registers (all T threads of the workgroup take
// part; `red` is T/64 words of LDS). Pieces of slots past the valid ones and pairs past the block
// are masked out of the maximum, and their codes are cleared. The block maximum of |x| is taken
// over fp16 bit patterns: without the sign bit, the order of the patterns of numbers is the order
// of their magnitudes, and a NaN pattern exceeds every number, so a NaN among the values gives a
// NaN maximum (and scale).
template <int FMT, int NL, int T>
__device__ __forceinline__ void encode_unit(const uint4 (&x)[NL], const CompUnit &u,
                                            int32_t pieces, int32_t rpp, uint32_t *red) {
  uint32_t mx = 0u;
  uint32_t keep_bits = 0u;  // bit i: piece pair i is in the block and in a valid slot
#pragma unroll
  for (int i = 0; i < NL / 2; ++i) {
    const int32_t c = 2 * (threadIdx.x + i * T);
    const bool keep = c < pieces && (c / rpp) % kBlock < u.n;
    keep_bits |= static_cast<uint32_t>(keep) << i;
    const uint32_t am = keep ? 0x7FFF7FFFu : 0u;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const uint4 &y = x[2 * i + k];
      mx = max_u16x2(mx, y.x & am);
      mx = max_u16x2(mx, y.y & am);
      mx = max_u16x2(mx, y.z & am);
      mx = max_u16x2(mx, y.w & am);
    }
  }
  uint32_t m = max(mx & 0xFFFFu, mx >> 16);
  for (int off = 32; off > 0; off >>= 1) m = max(m, static_cast<uint32_t>(__shfl_xor(m, off)));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = red[0];
#pragma unroll
  for (int w = 1; w < T / 64; ++w) m = max(m, red[w]);
  const float amax = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(m)));
  const float sc = amax / Q8<FMT>::kMax;
  // one of two loops, chosen once per unit
  if (sc > 0.f && sc < __builtin_inff())
    encode_pairs<FMT, NL, T, true>(x, keep_bits, pieces, u.dp, sc);
  else
    encode_pairs<FMT, NL, T, false>(x, keep_bits, pieces, u.dp, sc);
  if (threadIdx.x == 0) *u.scale = sc;
}

// One workgroup of T threads per unit (blocks of more than 8192 pieces).
template <int FMT, int NL, int T>
__global__ void __launch_bounds__(T) compress_f16_regs_kernel(const CompArgs a) {
  __shared__ uint32_t red[T / 64];
  const CompUnit u = comp_unit(a, blockIdx.x);
  if (!u.ok) return;
  const int32_t pieces = a.H * kBlock * a.D / 8;
  uint4 x[NL];
  load_pieces<NL, T>(u.sp, pieces, x);
  encode_unit<FMT, NL, T>(x, u, pieces, a.D / 8, red);
}

// One workgroup of 512 threads per CU walks units blockIdx.x, + gridDim.x, ...: the loads of its
// next unit are issued before the current one is encoded, into the other of two register sets,
// so they stay in flight while it encodes and stores. (A workgroup per unit loads, then encodes:
// its loads and its encoding never overlap, and a read-only kernel of that shape reaches only
// about 5.8 TB/s.) The two halves of the loop reduce through separate LDS words: a wavefront
// reaching one half's reduction has passed the other half's barrier, which every wavefront
// reaches only after reading the words of the reduction before it. A skipped unit still takes
// that barrier, so the alternation holds whichever units are skipped.
template <int FMT, int NL>
__global__ void __launch_bounds__(512) compress_f16_stream_kernel(const CompArgs a) {
  constexpr int T = 512;
  __shared__ uint32_t red[2][T / 64];
  const int32_t pieces = a.H * kBlock * a.D / 8;
  const int32_t rpp = a.D / 8;
  int32_t u = blockIdx.x;
  if (u >= a.n_units) return;
  // Loads are issued unconditionally (after the last unit, that unit again stands in, and is not
  // encoded twice): a register set loaded on one path only would be merged across the loop edge
  // with copies that wait for every load in flight.
  uint4 xa[NL], xb[NL];
  CompUnit ua = comp_unit(a, u), ub;
  load_pieces<NL, T>(ua.sp, pieces, xa);
  for (;;) {
    const int32_t u1 = u + gridDim.x;  // uniform over the workgroup, as every test below
    const bool more1 = u1 < a.n_units;
    ub = comp_unit(a, more1 ? u1 : u);
    load_pieces<NL, T>(ub.sp, pieces, xb);
    if (ua.ok)
      encode_unit<FMT, NL, T>(xa, ua, pieces, rpp, red[0]);
    else
      __syncthreads();
    if (!more1) break;
    u = u1 + gridDim.x;
    const bool more2 = u < a.n_units;
    ua = comp_unit(a, more2 ? u : u1);
    load_pieces<NL, T>(ua.sp, pieces, xa);
    if (ub.ok)
      encode_unit<FMT, NL, T>(xb, ub, pieces, rpp, red[1]);
    else
      __syncthreads();
    if (!more2) break;
  }
}

}  // namespace kvc

using namespace kvc;

extern "C" {

kvc_status kvc_append_contig(void *k_cache, void *v_cache, kvc_dtype dtype, int32_t B, int32_t H,
                             int32_t S_max, int32_t D, const int32_t *pos, int32_t n_tok,
                             const void *k_new, const void *v_new, void *stream) {
  if (B < 0 || H < 1 || S_max < 0 || n_tok < 0) return KVC_E_INVALID;
  if (!is_f32_or_f16(dtype)) return KVC_E_UNSUPPORTED;
  if (D != 64 && D != 128) return KVC_E_UNSUPPORTED;
  if (B == 0 || n_tok == 0) return KVC_OK;
  if (!k_cache || !v_cache || !pos || !k_new || !v_new) return KVC_E_INVALID;
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_new) || !aligned16(v_new))
    return KVC_E_INVALID;
  const int32_t row_bytes = D * elt_bytes(dtype);
  const int64_t threads = static_cast<int64_t>(B) * n_tok * H * (row_bytes / 16);
  const int64_t grid = (threads + kThreads - 1) / kThreads;
  if (grid > INT32_MAX) return KVC_E_INVALID;
  hipLaunchKernelGGL(append_contig_kernel, dim3(static_cast<uint32_t>(grid)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<char *>(k_cache),
                     static_cast<char *>(v_cache), static_cast<const char *>(k_new),
                     static_cast<const char *>(v_new), pos, B, H, S_max, n_tok, row_bytes);
  return launch_status();
}

static kvc_status check_layer(const kvc_paged_layer *L) {
  if (!L || L->num_blocks < 1 || L->num_heads < 1) return KVC_E_INVALID;
  if (L->head_dim != 64 && L->head_dim != 128) return KVC_E_UNSUPPORTED;
  if (L->kv_dtype != KVC_F32 && L->kv_dtype != KVC_F16 && !is_q8(L->kv_dtype))
    return KVC_E_UNSUPPORTED;
  if (!L->k_pool || !L->v_pool || !aligned16(L->k_pool) || !aligned16(L->v_pool))
    return KVC_E_INVALID;
  if (is_q8(L->kv_dtype) && (!L->k_scale || !L->v_scale)) return KVC_E_INVALID;
  return KVC_OK;
}

kvc_status kvc_copy_blocks(const kvc_paged_layer *layer, const int32_t *src, const int32_t *dst,
                           int32_t n, void *stream) {
  kvc_status st = check_layer(layer);
  if (st != KVC_OK) return st;
  if (n < 0) return KVC_E_INVALID;
  if (n == 0) return KVC_OK;
  if (!src || !dst) return KVC_E_INVALID;
  const int64_t block_bytes = static_cast<int64_t>(layer->num_heads) * kBlock * layer->head_dim *
                              elt_bytes(layer->kv_dtype);
  const bool fp8 = is_q8(layer->kv_dtype);
  const int64_t slices = (block_bytes / 16 + kCopyPieces - 1) / kCopyPieces;
  const int64_t grid = static_cast<int64_t>(n) * slices;
  if (grid > INT32_MAX) return KVC_E_INVALID;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(static_cast<uint32_t>(grid)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<char *>(layer->k_pool),
                     static_cast<char *>(layer->v_pool), fp8 ? layer->k_scale : nullptr,
                     fp8 ? layer->v_scale : nullptr, src, dst, layer->num_blocks, block_bytes,
                     static_cast<int32_t>(slices));
  return launch_status();
}

kvc_status kvc_write_paged(const kvc_paged_layer *layer, const int64_t *slots, int32_t n_tok,
                           const void *k_new, const void *v_new, kvc_dtype new_dtype,
                           void *stream) {
  kvc_status st = check_layer(layer);
  if (st != KVC_OK) return st;
  if (n_tok < 0) return KVC_E_INVALID;
  if (n_tok == 0) return KVC_OK;
  if (!slots || !k_new || !v_new || !aligned16(k_new) || !aligned16(v_new)) return KVC_E_INVALID;
  const int32_t H = layer->num_heads, D = layer->head_dim;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (is_q8(layer->kv_dtype)) {
    if (!is_f32_or_f16(new_dtype)) return KVC_E_UNSUPPORTED;
    auto *kp = static_cast<uint8_t *>(layer->k_pool);
    auto *vp = static_cast<uint8_t *>(layer->v_pool);
    const bool f16 = new_dtype == KVC_F16;
    auto kern = layer->kv_dtype == KVC_E4M3
                    ? (f16 ? write_paged_q8_kernel<true, KVC_E4M3> : write_paged_q8_kernel<false, KVC_E4M3>)
                    : (f16 ? write_paged_q8_kernel<true, KVC_I8> : write_paged_q8_kernel<false, KVC_I8>);
    hipLaunchKernelGGL(kern, dim3(n_tok), dim3(kThreads), 0, s, kp, vp, layer->k_scale,
                       layer->v_scale, k_new, v_new, slots, n_tok, H, D, layer->num_blocks);
    return launch_status();
  }
  if (new_dtype != layer->kv_dtype) return KVC_E_UNSUPPORTED;
  const int32_t row_bytes = D * elt_bytes(layer->kv_dtype);
  const int64_t threads = static_cast<int64_t>(n_tok) * H * (row_bytes / 16);
  const int64_t grid = (threads + kThreads - 1) / kThreads;
  if (grid > INT32_MAX) return KVC_E_INVALID;
  hipLaunchKernelGGL(write_paged_kernel, dim3(static_cast<uint32_t>(grid)), dim3(kThreads), 0, s,
                     static_cast<char *>(layer->k_pool), static_cast<char *>(layer->v_pool),
                     static_cast<const char *>(k_new), static_cast<const char *>(v_new), slots,
                     n_tok, H, layer->num_blocks, row_bytes);
  return launch_status();
}

kvc_status kvc_compress_blocks(const kvc_paged_layer *src, const kvc_paged_layer *dst,
                               const int32_t *src_ids, const int32_t *dst_ids,
                               const int32_t *n_valid, int32_t n, void *stream) {
  kvc_status st = check_layer(src);
  if (st != KVC_OK) return st;
  st = check_layer(dst);
  if (st != KVC_OK) return st;
  if (!is_f32_or_f16(src->kv_dtype) || !is_q8(dst->kv_dtype)) return KVC_E_UNSUPPORTED;
  if (src->num_heads != dst->num_heads || src->head_dim != dst->head_dim) return KVC_E_INVALID;
  if (static_cast<int64_t>(src->num_heads) * kBlock * src->head_dim > (int64_t{1} << 30))
    return KVC_E_INVALID;  // element offsets within a block stay 32-bit
  if (n < 0) return KVC_E_INVALID;
  if (n == 0) return KVC_OK;
  if (!src_ids || !dst_ids) return KVC_E_INVALID;
  const bool f16 = src->kv_dtype == KVC_F16;
  const bool e4m3 = dst->kv_dtype == KVC_E4M3;
  const int64_t pieces = static_cast<int64_t>(src->num_heads) * kBlock * src->head_dim / 8;
  if (f16 && pieces <= kCompMaxPieces) {
    if (static_cast<int64_t>(n) * 2 > INT32_MAX) return KVC_E_INVALID;
    const CompArgs ca{static_cast<const char *>(src->k_pool), static_cast<const char *>(src->v_pool),
                      static_cast<uint8_t *>(dst->k_pool), static_cast<uint8_t *>(dst->v_pool),
                      dst->k_scale, dst->v_scale, src_ids, dst_ids, n_valid, src->num_heads,
                      src->head_dim, src->num_blocks, dst->num_blocks, n * 2};
    hipStream_t s = static_cast<hipStream_t>(stream);
    using K = void (*)(CompArgs);
    if (pieces > 16 * 512) {  // 16 pieces per thread at 1024 threads, a workgroup per unit
      const K kr = e4m3 ? compress_f16_regs_kernel<KVC_E4M3, 16, 1024>
                        : compress_f16_regs_kernel<KVC_I8, 16, 1024>;
      hipLaunchKernelGGL(kr, dim3(static_cast<uint32_t>(n) * 2), dim3(1024), 0, s, ca);
      return launch_status();
    }
    // pieces per thread at 512 threads: 4, 8 or 16; one streaming workgroup per CU
    const K e4[] = {compress_f16_stream_kernel<KVC_E4M3, 4>,
                    compress_f16_stream_kernel<KVC_E4M3, 8>,
                    compress_f16_stream_kernel<KVC_E4M3, 16>};
    const K i8[] = {compress_f16_stream_kernel<KVC_I8, 4>, compress_f16_stream_kernel<KVC_I8, 8>,
                    compress_f16_stream_kernel<KVC_I8, 16>};
    const int sel = pieces <= 4 * 512 ? 0 : pieces <= 8 * 512 ? 1 : 2;
    const int64_t grid = std::min<int64_t>(static_cast<int64_t>(n) * 2, device_cu_count());
    hipLaunchKernelGGL(e4m3 ? e4[sel] : i8[sel], dim3(static_cast<uint32_t>(grid)), dim3(512), 0,
                       s, ca);
    return launch_status();
  }
  auto kern = e4m3 ? (f16 ? compress_blocks_kernel<true, KVC_E4M3>
                          : compress_blocks_kernel<false, KVC_E4M3>)
                   : (f16 ? compress_blocks_kernel<true, KVC_I8>
                          : compress_blocks_kernel<false, KVC_I8>);
  hipLaunchKernelGGL(kern, dim3(n), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     src->k_pool, src->v_pool, static_cast<uint8_t *>(dst->k_pool),
                     static_cast<uint8_t *>(dst->v_pool), dst->k_scale, dst->v_scale, src_ids,
                     dst_ids, n_valid, src->num_heads, src->head_dim, src->num_blocks,
                     dst->num_blocks);
  return launch_status();
}

}  // extern "C"
