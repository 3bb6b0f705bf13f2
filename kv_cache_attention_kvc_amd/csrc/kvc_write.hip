// Cache writes for gfx950: contiguous append, paged scatter, 8-bit (fp8-e4m3 or int8) per-block
// quantised writes, and copy-on-write block copies.
//
// The new token's K/V are stored before attention reads the cache ("LLM Inference Acceleration
// -- KV Cache", section 3.1). Paged writes go to slot = block*16 + offset chosen by the host pool
// ("KV Cache and PagedAttention", sections 3.1 and 3.3). 8-bit pools hold OCP e4m3 or int8 codes
// with one fp32 scale per block for K and one for V ("KV Cache Mechanism Explained", section 8,
// item 3: FP8/INT8 history with a scaling factor; "KV Cache and PagedAttention", section 7.2).
#include "kvc_internal.h"

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

// One workgroup per copy pair: the whole block (all heads) of K and V, and the fp8 scales.
__global__ void __launch_bounds__(kThreads)
copy_blocks_kernel(char *kp, char *vp, float *ks, float *vs, const int32_t *src,
                   const int32_t *dst, int32_t num_blocks, int64_t block_bytes) {
  const int32_t s = src[blockIdx.x];
  const int32_t d = dst[blockIdx.x];
  if (static_cast<uint32_t>(s) >= static_cast<uint32_t>(num_blocks) ||
      static_cast<uint32_t>(d) >= static_cast<uint32_t>(num_blocks) || s == d)
    return;
  const int64_t chunks = block_bytes / 16;
  const int64_t so = static_cast<int64_t>(s) * block_bytes;
  const int64_t dof = static_cast<int64_t>(d) * block_bytes;
  for (int64_t c = threadIdx.x; c < chunks; c += kThreads) {
    *reinterpret_cast<uint4 *>(kp + dof + c * 16) = *reinterpret_cast<const uint4 *>(kp + so + c * 16);
    *reinterpret_cast<uint4 *>(vp + dof + c * 16) = *reinterpret_cast<const uint4 *>(vp + so + c * 16);
  }
  if (threadIdx.x == 0 && ks) {
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
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(n), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<char *>(layer->k_pool),
                     static_cast<char *>(layer->v_pool), fp8 ? layer->k_scale : nullptr,
                     fp8 ? layer->v_scale : nullptr, src, dst, layer->num_blocks, block_bytes);
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

}  // extern "C"
