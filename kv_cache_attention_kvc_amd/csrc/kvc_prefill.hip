// Chunked prefill attention over a contiguous or paged KV cache, on the matrix cores (gfx950).
//
// Sequence b brings a chunk of n_b new tokens, the last n_b of its L_b positions, whose K and V
// are already in the cache. Row i of the chunk (position P = L_b - n_b + i) attends positions
// 0 .. P: the causal mask of a forward pass over several tokens at start_pos L_b - n_b ("LLM
// Inference Acceleration -- KV Cache", section 3.1, triu(-inf, start_pos + 1) when more than one
// token enters). Blocks are gathered through the block table and the attention inside a block
// is tiled in on-chip memory ("KV Cache and PagedAttention", section 5.3: FlashAttention within
// blocks, PagedAttention between them; "LLM Inference Acceleration -- KV Cache", section 6.3).
//
// A workgroup of four wavefronts takes one K/V head and 64 query rows: 64 consecutive positions
// of one query head, or 32 positions of 2 heads, or 16 positions of 4 heads of a group sharing
// the K/V head. It walks the 16-position key blocks from 0 to its last row's position. Each
// block's K and V is loaded once, by all 256 threads with 16-byte loads, into LDS (two buffers,
// one barrier per block) and serves the four wavefronts. Per wavefront and block the arithmetic
// is that of grouped decode with 16 query rows in place of 16 query heads:
//   S^T = K . Q^T with D/32 v_mfma_f32_16x16x32_f16: lane (g, j) = (lane/16, lane%16) feeds key
//     row j (from LDS) and query row j (registers) and receives the scores of keys 4g..4g+3 for
//     row j; keys past the row's position are masked to -inf;
//   the online softmax keeps, per row, a reference that moves only when a block's maximum passes
//     it by the headroom, and per lane the partial sum of its keys' weights;
//   O^T = V^T . P^T with D/16 x 2 v_mfma_f32_16x16x16_f16, the weights as fp16 hi + lo (about 22
//     bits) and V^T read from LDS one fp16 at a time.
// LDS layouts: K rows keep their 16-byte columns XOR-swizzled by the row index (the 16 rows a
// read instruction takes land on distinct banks); V rows are swizzled by row group as in decode.
#include <algorithm>

#include "kvc_internal.h"
#include "kvc_wave.h"

namespace kvc {

constexpr int kPfWaves = 4;
constexpr int kPfThreads = kPfWaves * kWave;
constexpr int kPfRows = 16 * kPfWaves;  // query rows per workgroup
constexpr int kMaxSeqs = 4096;
// weight headroom (log2 units): weights stay below 2^kHi, so both fp16 terms stay finite
constexpr float kHead = 7.f;
constexpr float kHi = 15.f;

struct PrefillArgs {
  const char *q;  // fp16 [total][Hq][D]
  const char *k;  // paged: [num_blocks][H][16][D]; contiguous: [B][H][S_max][D] (fp16)
  const char *v;
  const int32_t *tables;
  const int32_t *q_start;  // [B+1]
  const int32_t *lens;     // [B]
  void *out;               // [total][Hq][D]
  int64_t seq_stride;      // contiguous: S_max
  int32_t B, H, G, Hq, cap, mbps, num_blocks, total;
  int32_t gh;  // query heads per workgroup (1, 2 or 4); positions per workgroup = 64 / gh
  int32_t out_f16;
  float cl2;   // scale * log2(e)
};

// Row range [r0, r0 + n) of sequence b's chunk, clamped so that it lies inside [0, total) and
// holds at most L_b rows; L_b clamped to [0, cap].
struct Chunk {
  int32_t r0, n, L;
};

static __device__ __forceinline__ Chunk chunk_of(const PrefillArgs &a, int32_t b) {
  Chunk c;
  c.L = min(max(a.lens[b], 0), a.cap);
  const int32_t lo = min(max(a.q_start[b], 0), a.total);
  const int32_t hi = min(max(a.q_start[b + 1], lo), a.total);
  c.r0 = lo;
  c.n = min(hi - lo, c.L);
  return c;
}

// pre[b] = workgroups before sequence b along x (ceil(n_b / pt) each), pre[B] = total, in LDS.
static __device__ void tile_prefix(const PrefillArgs &a, int32_t pt, int32_t *pre, int32_t *wsum) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid >> 6;
  const int per = (a.B + kPfThreads - 1) / kPfThreads;
  const int lo = min(a.B, tid * per);
  const int hi = min(a.B, lo + per);
  int32_t sum = 0;
  for (int i = lo; i < hi; ++i) sum += (chunk_of(a, i).n + pt - 1) / pt;
  int32_t inc = sum;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int32_t v = __shfl_up(inc, off);
    if (lane >= off) inc += v;
  }
  if (lane == kWave - 1) wsum[wave] = inc;
  __syncthreads();
  for (int w = 0; w < wave; ++w) inc += wsum[w];
  int32_t run = inc - sum;
  for (int i = lo; i < hi; ++i) {
    pre[i] = run;
    run += (chunk_of(a, i).n + pt - 1) / pt;
  }
  if (tid == kPfThreads - 1) pre[a.B] = inc;
  __syncthreads();
}

template <bool PAGED, int D>
__global__ void __launch_bounds__(kPfThreads) prefill_kernel(const PrefillArgs a) {
  constexpr int ROW = D * 2;         // bytes of one fp16 row
  constexpr int NCH = D / 8;         // 16-byte columns per row
  constexpr int BLK = kBlock * ROW;  // bytes of one block of K (or V)
  constexpr int NQK = D / 32;        // score MFMAs per block
  constexpr int NDC = D / 16;        // 16-dim output blocks
  extern __shared__ int32_t smem[];
  int32_t *pre = smem;
  int32_t *wsum = smem + a.B + 1;
  char *kv_lds = reinterpret_cast<char *>(smem) + ((a.B + 1 + kPfWaves + 3) / 4) * 16;
  // kv_lds: [2 buffers][K block | V block]

  const int32_t pt = kPfRows / a.gh;
  tile_prefix(a, pt, pre, wsum);
  const int32_t x = blockIdx.x;
  if (x >= pre[a.B]) return;
  // the sequence of workgroup x: the largest b with pre[b] <= x
  int32_t lo = 0, hi = a.B - 1;
  while (lo < hi) {
    const int32_t mid = (lo + hi + 1) >> 1;
    if (pre[mid] <= x) lo = mid; else hi = mid - 1;
  }
  const int32_t b = lo;
  const Chunk ch = chunk_of(a, b);
  const int32_t ntile = (ch.n + pt - 1) / pt;
  const int32_t tile = ntile - 1 - (x - pre[b]);  // the longest tiles of a sequence start first
  const int32_t rt0 = tile * pt;                  // chunk-relative rows of the workgroup
  const int32_t rt1 = min(rt0 + pt, ch.n);
  const int32_t base_pos = ch.L - ch.n;           // position of chunk row 0

  const int32_t nsub = a.G / a.gh;
  const int32_t hk = blockIdx.y / nsub;
  const int32_t hq0 = hk * a.G + (blockIdx.y % nsub) * a.gh;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int w = tid >> 6;
  const int g = lane >> 4;
  const int j = lane & 15;
  const int32_t hq = hq0 + w % a.gh;
  const int32_t rw0 = rt0 + 16 * (w / a.gh);      // the wavefront's first row
  const int32_t nrow = max(0, min(16, rt1 - rw0));
  const int32_t wave_last = base_pos + rw0 + nrow - 1;  // its last row's position
  const int32_t last_pos = base_pos + rt1 - 1;          // the workgroup's
  const int32_t nkb = last_pos / kBlock + 1;

  // q operand: row j of the wavefront (rows past its end repeat its last row; a wavefront with
  // no rows reads the workgroup's first row and stores nothing), 8 dims per MFMA
  const int32_t my_rel = nrow > 0 ? rw0 + min(j, nrow - 1) : rt0;
  uint4 qv[NQK];
  {
    const char *qr = a.q + (static_cast<int64_t>(ch.r0 + my_rel) * a.Hq + hq) * ROW;
#pragma unroll
    for (int c = 0; c < NQK; ++c) qv[c] = *reinterpret_cast<const uint4 *>(qr + (g + 4 * c) * 16);
  }
  const int32_t my_pos = base_pos + my_rel;

  // block loads: thread t < 16*NCH takes 16-byte column t % NCH of key row t / NCH
  const bool loader = tid < kBlock * NCH;
  const int kr = tid / NCH;
  const int kc = tid % NCH;
  const int64_t kv_head_off = PAGED ? static_cast<int64_t>(hk) * BLK
                                    : (static_cast<int64_t>(b) * a.H + hk) * a.seq_stride * ROW;
  auto load_block = [&](int32_t kb, uint4 &kreg, uint4 &vreg) -> bool {
    // rows past the sequence's end read its last row (finite; those keys are masked)
    const int32_t row = min(kb * kBlock + kr, ch.L - 1);
    int64_t off;
    bool ok = true;
    if constexpr (PAGED) {
      const int32_t phys = __builtin_amdgcn_readfirstlane(a.tables[static_cast<int64_t>(b) * a.mbps + kb]);
      ok = static_cast<uint32_t>(phys) < static_cast<uint32_t>(a.num_blocks);
      const int32_t sp = ok ? phys : 0;
      off = static_cast<int64_t>(sp) * a.H * BLK + kv_head_off + (row - kb * kBlock) * ROW;
    } else {
      off = kv_head_off + static_cast<int64_t>(row) * ROW;
    }
    if (loader) {
      kreg = load_stream(a.k + off + kc * 16);
      vreg = load_stream(a.v + off + kc * 16);
    }
    return ok;
  };
  auto store_block = [&](int buf, const uint4 &kreg, const uint4 &vreg) {
    if (!loader) return;
    char *kb_lds = kv_lds + buf * 2 * BLK;
    char *vb_lds = kb_lds + BLK;
    *reinterpret_cast<uint4 *>(kb_lds + kr * ROW + ((kc ^ (kr & (NCH - 1))) * 16)) = kreg;
    *reinterpret_cast<uint4 *>(vb_lds + kr * ROW + ((kc ^ (2 * ((kr >> 2) & 3))) * 16)) = vreg;
  };

  f32x4 o[NDC];
#pragma unroll
  for (int dc = 0; dc < NDC; ++dc) o[dc] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = kFloor, l = 0.f;

  uint4 kreg = make_uint4(0, 0, 0, 0), vreg = make_uint4(0, 0, 0, 0);
  bool ok_cur = load_block(0, kreg, vreg);
  for (int32_t kb = 0; kb < nkb; ++kb) {
    store_block(kb & 1, kreg, vreg);
    const bool ok = ok_cur;
    if (kb + 1 < nkb) ok_cur = load_block(kb + 1, kreg, vreg);
    __syncthreads();
    // a wavefront whose rows all precede this block, or a block id outside the pool: skip
    if (nrow == 0 || kb * kBlock > wave_last || !ok) continue;
    const char *kb_lds = kv_lds + (kb & 1) * 2 * BLK;
    const _Float16 *vb_lds = reinterpret_cast<const _Float16 *>(kb_lds + BLK);
    f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NQK; ++c) {
      const uint4 kv = *reinterpret_cast<const uint4 *>(kb_lds + j * ROW +
                                                        (((g + 4 * c) ^ (j & (NCH - 1))) * 16));
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(kv), as_f16x8(qv[c]), sacc, 0, 0, 0);
    }
    float xs[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      xs[e] = kb * kBlock + 4 * g + e <= my_pos ? sacc[e] * a.cl2 : -__builtin_inff();
    float mx = fmaxf(fmaxf(xs[0], xs[1]), fmaxf(xs[2], xs[3]));
    {
      float u, v;
      lane_pair<16>(mx, u, v);
      mx = fmaxf(u, v);
      lane_pair<32>(mx, u, v);
      mx = fmaxf(u, v);
    }
    const bool up = mx > m + kHi;
    if (__ballot(up) != 0) {
      const float mnew = up ? mx - kHead : m;
      const float f = __builtin_amdgcn_exp2f(m - mnew);
      l *= f;
#pragma unroll
      for (int dc = 0; dc < NDC; ++dc) o[dc] *= f;
      m = mnew;
    }
    f16x4 ph, pl;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float p = __builtin_amdgcn_exp2f(xs[e] - m);
      l += p;
      ph[e] = static_cast<_Float16>(p);
      pl[e] = static_cast<_Float16>(p - static_cast<float>(ph[e]));
    }
    const _Float16 *vr = vb_lds + (4 * g) * D + (j & 7);
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) {
      const int col = (2 * dc + (j >> 3)) ^ (2 * g);
      f16x4 va;
#pragma unroll
      for (int e = 0; e < 4; ++e) va[e] = vr[e * D + col * 8];
      o[dc] = __builtin_amdgcn_mfma_f32_16x16x16f16(va, ph, o[dc], 0, 0, 0);
      o[dc] = __builtin_amdgcn_mfma_f32_16x16x16f16(va, pl, o[dc], 0, 0, 0);
    }
  }
  if (nrow == 0) return;
  float u, v;
  lane_pair<16>(l, u, v);
  l = u + v;
  lane_pair<32>(l, u, v);
  l = u + v;
  if (j >= nrow) return;
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  const int64_t orow = (static_cast<int64_t>(ch.r0 + rw0 + j) * a.Hq + hq) * D;
#pragma unroll
  for (int dc = 0; dc < NDC; ++dc) {
    const int64_t i = orow + 16 * dc + 4 * g;
    const f32x4 r = o[dc] * inv;
    if (a.out_f16) {
      const f16x4 h = {static_cast<_Float16>(r[0]), static_cast<_Float16>(r[1]),
                       static_cast<_Float16>(r[2]), static_cast<_Float16>(r[3])};
      *reinterpret_cast<f16x4 *>(static_cast<_Float16 *>(a.out) + i) = h;
    } else {
      *reinterpret_cast<f32x4 *>(static_cast<float *>(a.out) + i) = r;
    }
  }
}

using PrefillKernel = void (*)(PrefillArgs);

template <bool PAGED>
static PrefillKernel pick_prefill(int D) {
  if (D == 64) return prefill_kernel<PAGED, 64>;
  if (D == 128) return prefill_kernel<PAGED, 128>;
  return nullptr;
}

// Shared validation and launch. cap: positions a sequence can hold.
static kvc_status launch_prefill(bool paged, PrefillArgs &a, int32_t D, kvc_dtype q_dtype,
                                 kvc_dtype kv_dtype, kvc_dtype out_dtype, float scale,
                                 void *stream) {
  if (a.B < 0 || a.B > kMaxSeqs || a.H < 1 || a.G < 1 || a.total < 0 || a.cap < 0)
    return KVC_E_INVALID;
  if (static_cast<int64_t>(a.H) * a.G > (1 << 20)) return KVC_E_INVALID;
  if (q_dtype != KVC_F16 || kv_dtype != KVC_F16) return KVC_E_UNSUPPORTED;
  if (out_dtype != KVC_F16 && out_dtype != KVC_F32) return KVC_E_UNSUPPORTED;
  if (D != 64 && D != 128) return KVC_E_UNSUPPORTED;
  if (!(scale == scale) || __builtin_isinf(scale)) return KVC_E_INVALID;
  if (a.B == 0 || a.total == 0) return KVC_OK;
  if (!a.q || !a.out || !a.q_start || !a.lens || !a.k || !a.v) return KVC_E_INVALID;
  if (!aligned16(a.q) || !aligned16(a.out) || !aligned16(a.k) || !aligned16(a.v))
    return KVC_E_INVALID;
  a.Hq = a.H * a.G;
  a.gh = a.G % 4 == 0 ? 4 : (a.G % 2 == 0 ? 2 : 1);
  a.out_f16 = out_dtype == KVC_F16;
  a.cl2 = scale * kLog2e;
  const int32_t pt = kPfRows / a.gh;
  // an upper bound on the workgroups along x: sum_b ceil(n_b / pt) <= total / pt + B
  const int64_t gx = (static_cast<int64_t>(a.total) + pt - 1) / pt + a.B;
  const int64_t gy = static_cast<int64_t>(a.H) * (a.G / a.gh);
  if (gx > INT32_MAX || gy > 65535) return KVC_E_INVALID;
  const size_t shmem = static_cast<size_t>((a.B + 1 + kPfWaves + 3) / 4) * 16 +
                       static_cast<size_t>(2) * 2 * kBlock * D * 2;
  PrefillKernel kern = paged ? pick_prefill<true>(D) : pick_prefill<false>(D);
  if (!kern) return KVC_E_UNSUPPORTED;
  hipLaunchKernelGGL(kern, dim3(static_cast<uint32_t>(gx), static_cast<uint32_t>(gy)),
                     dim3(kPfThreads), shmem, static_cast<hipStream_t>(stream), a);
  return launch_status();
}

}  // namespace kvc

using namespace kvc;

extern "C" {

kvc_status kvc_prefill_contig(const void *q, kvc_dtype q_dtype, int32_t G, const void *k_cache,
                              const void *v_cache, kvc_dtype kv_dtype, const int32_t *q_start,
                              const int32_t *ctx_lens, int32_t B, int32_t H_kv, int32_t S_max,
                              int32_t D, int32_t total_q, float scale, void *out,
                              kvc_dtype out_dtype, void *stream) {
  if (S_max < 0) return KVC_E_INVALID;
  PrefillArgs a{};
  a.q = static_cast<const char *>(q);
  a.k = static_cast<const char *>(k_cache);
  a.v = static_cast<const char *>(v_cache);
  a.q_start = q_start;
  a.lens = ctx_lens;
  a.out = out;
  a.seq_stride = S_max;
  a.B = B;
  a.H = H_kv;
  a.G = G;
  a.cap = S_max;
  a.total = total_q;
  return launch_prefill(false, a, D, q_dtype, kv_dtype, out_dtype, scale, stream);
}

kvc_status kvc_prefill_paged(const void *q, kvc_dtype q_dtype, int32_t G,
                             const kvc_paged_layer *layer, const int32_t *block_tables,
                             int32_t max_blocks_per_seq, const int32_t *q_start,
                             const int32_t *ctx_lens, int32_t B, int32_t total_q, float scale,
                             void *out, kvc_dtype out_dtype, void *stream) {
  if (!layer || max_blocks_per_seq < 1 || max_blocks_per_seq > INT32_MAX / kBlock)
    return KVC_E_INVALID;
  if (layer->num_blocks < 1 || layer->num_heads < 1) return KVC_E_INVALID;
  if (B > 0 && total_q > 0 && !block_tables) return KVC_E_INVALID;
  PrefillArgs a{};
  a.q = static_cast<const char *>(q);
  a.k = static_cast<const char *>(layer->k_pool);
  a.v = static_cast<const char *>(layer->v_pool);
  a.tables = block_tables;
  a.q_start = q_start;
  a.lens = ctx_lens;
  a.out = out;
  a.B = B;
  a.H = layer->num_heads;
  a.G = G;
  a.cap = max_blocks_per_seq * kBlock;
  a.mbps = max_blocks_per_seq;
  a.num_blocks = layer->num_blocks;
  a.total = total_q;
  return launch_prefill(true, a, layer->head_dim, q_dtype, layer->kv_dtype, out_dtype, scale,
                        stream);
}

}  // extern "C"
