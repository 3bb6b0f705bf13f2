// Decode attention over a contiguous or paged KV cache, for gfx950 (64-lane wavefronts).
//
// out[b,h,:] = softmax(scale * q[b,h,:] . K[b,h,0:L_b,:]^T) . V[b,h,0:L_b,:]  -- one new query
// per sequence against every cached position, the new token included ("LLM Inference
// Acceleration -- KV Cache", section 3.1; "KV Cache Mechanism Explained", section 5.1). The
// paged layout gathers each sequence's 16-token blocks through its block table ("KV Cache and
// PagedAttention", section 3.2).
//
// Pass 1 (decode_partial_kernel). The work is the list of (sequence, head, block) triples in
// (h, b, block) order: H * sum_b ceil(L_b/16) tiles of 16 positions. It is cut into P equal
// contiguous chunks, one per wavefront, so every wavefront streams the same number of bytes
// whatever the length mix; each XCD takes a contiguous range of the chunks. A wavefront walks
// its chunk tile by tile with the next tile's loads in flight while it computes on the current
// one:
//   * a token row (D elements) is read by LPT lanes with 16-byte non-temporal loads (the K/V
//     stream is read once, so it is kept from displacing reusable lines), and one wave-wide load
//     covers TPL = 64/LPT consecutive rows (1 KiB contiguous); a tile takes LOADS such loads;
//   * each lane forms partial dot products over its 16 bytes of k; a butterfly of DPP adds
//     inside each LPT-lane group gives every lane of the group the full score;
//   * each group keeps its own online-softmax state (a reference m that moves only when a score
//     passes it by a fixed headroom, the sum l of the weights relative to it, and the
//     unnormalised output for the lane's 16-byte column), so the loop has no cross-group
//     traffic; the groups are combined once per (sequence, head) segment.
// Scores are kept in log2 units (multiplied by scale*log2(e)) and exponentials use v_exp_f32.
// A segment that covers a whole (sequence, head) is finished in place; a segment cut by a
// chunk boundary leaves (o[D], m, l) in one of the wavefront's two workspace records.
//
// Pass 2 (decode_merge_kernel). One wavefront per (sequence, head): pairs that were cut combine
// the records of the consecutive wavefronts that covered them, rescaling each by exp2 of its
// max minus the overall max; rows of empty sequences are zeroed; other pairs were finished in
// pass 1. Pass 1 leaves the chunk size and the per-sequence block prefix in the workspace, so
// pass 2 needs no other input. Stream order makes pass 1's stores visible to pass 2.
#include <mutex>
#include <vector>

#include "kvc_internal.h"
#include "kvc_wave.h"

namespace kvc {

typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr int kWgWaves = 4;
constexpr int kWgThreads = kWave * kWgWaves;
constexpr int kMaxWorkers = 8192;  // pass-1 wavefronts at most (records in a workspace)
constexpr int kMinChunk = 4;       // tiles per wavefront at least
constexpr int kPairTiles = 20;     // pair mode: tiles per wavefront at most
constexpr int kMfmaWgWaves = 4;    // matrix-core pass 1 with workgroup combine: wavefronts per CU
constexpr int kStageRows = 8;      // finished output rows a wavefront holds in LDS before storing
constexpr int kMaxGroup = 16;      // query heads one wavefront serves from one K/V head
constexpr int kMaxBatch = 4096;

// Workspace: [header int32[64] | prefix int32[B+1] | records float[kMaxWorkers][2][GQ][D+4]],
// each region 256-byte aligned. Header: chunk size C, and B, pairs per sequence, D, GQ of the
// pass-1 call, then whether pass 1 ran one workgroup per pair (nothing left to merge) and the
// work list's order (1: pair-major). GQ is the number of query heads a wavefront serves from
// one K/V head (1 for multi-head attention).
struct WsLayout {
  size_t pre_off, rec_off, total;
};

constexpr size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

constexpr WsLayout ws_layout(int B, int D, int GQ) {
  WsLayout l{};
  l.pre_off = 256;
  l.rec_off = l.pre_off + align256((static_cast<size_t>(B) + 1) * sizeof(int32_t));
  l.total = l.rec_off + static_cast<size_t>(kMaxWorkers) * 2 * GQ * (D + 4) * sizeof(float);
  return l;
}

// Workspace of kvc_decode_attn_paged_noalloc: a file-scope device array, one copy per GPU, held
// until the process ends, sized for the largest call that entry point takes (4096 sequences,
// D = 128, one query head per pair): 8,667,648 bytes. Host code never passes the array's name
// to a kernel (on the host it is only a stand-in for the symbol): it passes the device address
// that hipGetSymbolAddress returns for the current GPU.
constexpr size_t kScratchBytes = ws_layout(kMaxBatch, 128, 1).total;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

struct DecodeArgs {
  const void *q;
  const char *k;
  const char *v;
  const float *k_scale;
  const float *v_scale;
  const int32_t *tables;
  const int32_t *lens;
  const char *k_new;  // append mode: the new token's K and V, [B][H][D]; else null (H = K/V heads)
  const char *v_new;
  void *out;
  int32_t *ws_hdr;
  int32_t *ws_pre;
  float *ws_rec;
  int64_t seq_stride;  // contiguous: S_max
  int32_t B, H, cap, mbps, num_blocks, P, cmin;
  // shared K/V heads: G query heads per K/V head (q and out have Hq = H*G heads per sequence);
  // a pair is (sequence, K/V head, sub-group of GQ query heads), nsub = G/GQ pairs per K/V head
  // and Hp = H*nsub pairs per sequence. Multi-head attention: G = nsub = 1, Hp = Hq = H.
  int32_t G, nsub, Hp, Hq;
  int32_t gq;          // query heads per pair (G / nsub)
  int32_t window;      // rolling window: attend positions max(0, L - window) .. L-1 (0: none)
  int32_t stage_rows;  // staged output rows per wavefront (LDS)
  int32_t pair_mode;   // one workgroup per pair, combined in LDS (no merge), else equal chunks
  int32_t wg_combine;  // equal chunks; pairs cut between a workgroup's wavefronts combined in LDS
  int32_t pair_major;  // work-list order: pair-major, chunks XCD-contiguous (paged pools), else
                       // sequence-major, chunks round-robin over the XCDs (contiguous caches)
  int32_t q_f16, out_f16;
  float cl2;  // scale * log2(e)
};

// Sum over aligned groups of N lanes; every lane of a group gets the same bits.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp<0xB1>(x);  // quad_perm [1,0,3,2]: lane ^ 1
  x += dpp<0x4E>(x);  // quad_perm [2,3,0,1]: lane ^ 2
  if constexpr (N >= 8) x += dpp<0x141>(x);   // row_half_mirror: the other quad of 8
  if constexpr (N >= 16) x += dpp<0x140>(x);  // row_mirror: the other half of 16
  if constexpr (N >= 32) {
    float a, b;
    lane_pair<16>(x, a, b);  // the neighbouring row
    x = a + b;
  }
  return x;
}

__device__ __forceinline__ int32_t sread(const int32_t *p) {
  return __builtin_amdgcn_readfirstlane(*p);
}

// Load of a wave-uniform address through the scalar cache (read-only data: block tables). Its
// completion is counted apart from the vector loads, so waiting for it never waits for K/V.
typedef const __attribute__((address_space(4))) int32_t const_i32;
__device__ __forceinline__ int32_t sload(const int32_t *p) {
  return *(const_i32 *)(p);
}

// Unpack the 16 bytes a lane loaded into EPL floats.
template <int KV>
__device__ __forceinline__ void unpack(const uint4 &r, float *f) {
  if constexpr (KV == KVC_F32) {
    f[0] = __uint_as_float(r.x);
    f[1] = __uint_as_float(r.y);
    f[2] = __uint_as_float(r.z);
    f[3] = __uint_as_float(r.w);
  } else if constexpr (KV == KVC_F16) {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w[i])));
      f[2 * i + 1] =
          static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w[i] >> 16)));
    }
  } else if constexpr (KV == KVC_I8) {
    // exact through fp16 (see i8x4_to_f16); the fp16 values feed mixed-precision FMAs
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f16x2 lo, hi;
      i8x4_to_f16(w[i], lo, hi);
      f[4 * i + 0] = static_cast<float>(lo[0]);
      f[4 * i + 1] = static_cast<float>(lo[1]);
      f[4 * i + 2] = static_cast<float>(hi[0]);
      f[4 * i + 3] = static_cast<float>(hi[1]);
    }
  } else {
    // gfx950 converts OCP e4m3 in hardware (exact: every code is an fp32 value)
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w[i]), false);
      const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w[i]), true);
      f[4 * i + 0] = lo[0];
      f[4 * i + 1] = lo[1];
      f[4 * i + 2] = hi[0];
      f[4 * i + 3] = hi[1];
    }
  }
}

__device__ __forceinline__ float half_lo(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w)));
}
__device__ __forceinline__ float half_hi(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w >> 16)));
}

// N consecutive q elements (fp16 or fp32) starting at element i, loaded as raw 32-bit words with
// 8- or 16-byte vector loads and no branches (so the loads of a slice are all in flight together).
// The words are converted only when the slice is used, so the load is never waited for early.
template <bool QF16, int N>
struct QWords {
  static constexpr int W = QF16 ? N / 2 : N;
  uint32_t w[W];
};

template <bool QF16, int N>
__device__ __forceinline__ void load_q_words(const void *p, int64_t i, QWords<QF16, N> &q) {
  constexpr int W = QWords<QF16, N>::W;
  const char *b = static_cast<const char *>(p) + i * (QF16 ? 2 : 4);
  if constexpr (W % 4 == 0) {
#pragma unroll
    for (int k = 0; k < W / 4; ++k) {
      const uint4 r = reinterpret_cast<const uint4 *>(b)[k];
      q.w[4 * k] = r.x;
      q.w[4 * k + 1] = r.y;
      q.w[4 * k + 2] = r.z;
      q.w[4 * k + 3] = r.w;
    }
  } else {
    static_assert(W == 2, "q slices are 8 bytes or a multiple of 16");
    const uint2 r = *reinterpret_cast<const uint2 *>(b);
    q.w[0] = r.x;
    q.w[1] = r.y;
  }
}

template <bool QF16, int N>
__device__ __forceinline__ void q_floats(const QWords<QF16, N> &q, float *x) {
  if constexpr (QF16) {
#pragma unroll
    for (int u = 0; u < N / 2; ++u) {
      x[2 * u] = half_lo(q.w[u]);
      x[2 * u + 1] = half_hi(q.w[u]);
    }
  } else {
#pragma unroll
    for (int u = 0; u < N; ++u) x[u] = __uint_as_float(q.w[u]);
  }
}

// N consecutive output elements from floats, fp16 (round to nearest even) or fp32.
template <int N>
__device__ __forceinline__ void store_row(void *p, int64_t i, const float *x, float s, bool f16) {
  if (f16) {
    _Float16 h[N];
#pragma unroll
    for (int e = 0; e < N; ++e) h[e] = static_cast<_Float16>(x[e] * s);
    _Float16 *d = static_cast<_Float16 *>(p) + i;
#pragma unroll
    for (int e = 0; e < N; ++e) d[e] = h[e];
  } else {
    float *d = static_cast<float *>(p) + i;
#pragma unroll
    for (int e = 0; e < N; ++e) d[e] = x[e] * s;
  }
}

__device__ __forceinline__ void store_elem(void *p, int64_t i, float x, bool f16) {
  if (f16)
    reinterpret_cast<_Float16 *>(p)[i] = static_cast<_Float16>(x);
  else
    reinterpret_cast<float *>(p)[i] = x;
}

// ---- per-workgroup prefix of block counts ------------------------------------------------
// First logical block a sequence of length L attends under a rolling window (0 without one).
template <bool WIN>
__device__ __forceinline__ int32_t window_block(int32_t L, int32_t window) {
  if constexpr (WIN) return max(0, L - window) / kBlock;
  return 0;
}

// pre[b] = sum_{b' < b} nblk(b'), pre[B] = total blocks over sequences, and len[b] = clamp(L_b),
// all in LDS; nblk(b) = ceil(clamp(L_b)/16), less the blocks wholly before a rolling window.
// Each thread sums a run of consecutive sequences; runs are scanned with wave shuffles, then
// across the four waves through LDS.
template <bool WIN>
__device__ void block_prefix(const int32_t *lens, int B, int cap, int32_t window, int32_t *pre,
                             int32_t *len, int32_t *wsum) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid >> 6;
  const int per = (B + kWgThreads - 1) / kWgThreads;
  const int lo = min(B, tid * per);
  const int hi = min(B, lo + per);
  int32_t sum = 0;
  for (int i = lo; i < hi; ++i) {
    const int32_t L = min(max(lens[i], 0), cap);
    sum += (L + kBlock - 1) / kBlock - window_block<WIN>(L, window);
  }
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
    const int32_t L = min(max(lens[i], 0), cap);
    len[i] = L;
    run += (L + kBlock - 1) / kBlock - window_block<WIN>(L, window);
  }
  if (tid == kWgThreads - 1) pre[B] = inc;
  __syncthreads();
}

// ---- one tile: loads ---------------------------------------------------------------------
// Every fetch issues the same loads -- with one query head per wavefront the q slice of the
// tile's head first, then LOADS 16-byte loads of K and of V -- whatever the tile.
template <int KV, int D, bool QF16, int GQ>
struct TileRegs {
  using G = Geo<KV, D>;
  QWords<QF16, G::EPL> q[1];  // GQ == 1: this tile's q slice (unused otherwise)
  uint4 k[G::LOADS];
  uint4 v[G::LOADS];
  int32_t nt;       // valid rows (0: the tile contributes nothing)
  int32_t lo;       // rolling window: rows below lo lie before the window (first tile only)
  int32_t new_row;    // append mode: the row of the new token in this tile, else -1
  int32_t store_row;  // new_row if this wavefront stores it into the cache, else -1
  const char *kt;     // the tile's K and V in the cache (where the new row is stored)
  const char *vt;
  float ks, vs;     // fp8 block scales
};

// Tile j (logical block j) of K/V head hkv of sequence b (bkv = b*H + hkv); phys is its block id
// (paged); qrow is the row of q of the first query head the wavefront serves (loaded here when
// GQ == 1). live = false fetches a stand-in with nt = 0 (the first row of block 0 / of the
// sequence-head), for the step after a chunk's last tile.
template <bool PAGED, int KV, int D, bool QF16, int GQ, bool WIN>
__device__ __forceinline__ void fetch_tile(const DecodeArgs &a, TileRegs<KV, D, QF16, GQ> &t,
                                           int64_t bkv, int32_t hkv, int64_t qrow, int32_t j,
                                           int32_t phys, int32_t L, bool live, int g, int c) {
  using G = Geo<KV, D>;
  if constexpr (GQ == 1) load_q_words<QF16, G::EPL>(a.q, qrow * D + c * G::EPL, t.q[0]);
  const char *kt;
  const char *vt;
  bool valid = live;
  if constexpr (PAGED) {
    // addresses are formed from a clamped id, so nothing outside the pools is ever addressed
    valid = valid && static_cast<uint32_t>(phys) < static_cast<uint32_t>(a.num_blocks);
    const int32_t sp = valid ? phys : 0;
    const int64_t toff = (static_cast<int64_t>(sp) * a.H + hkv) * G::TILE;
    kt = a.k + toff;
    vt = a.v + toff;
    if constexpr (is_q8(KV)) {
      t.ks = valid ? a.k_scale[sp] : 0.f;
      t.vs = valid ? a.v_scale[sp] : 0.f;
    }
  } else {
    const int64_t toff = (bkv * a.seq_stride + static_cast<int64_t>(kBlock) * (valid ? j : 0)) *
                         G::ROW;
    kt = a.k + toff;
    vt = a.v + toff;
  }
  t.nt = valid ? min(kBlock, L - kBlock * j) : 0;
  // rolling window: positions before max(0, L - window) are not attended
  t.lo = WIN ? min(max(max(0, L - a.window) - kBlock * j, 0), kBlock) : 0;
  t.kt = kt;
  t.vt = vt;
  // append mode: the tile holding position L-1 takes that row from k_new/v_new (the lanes of
  // that row load from there instead of the cache) and stores it into the cache when consumed.
  // That tile is the last of its sequence-head, so it always takes the general path below and
  // the full-tile path carries no per-lane address choice.
  t.new_row = (a.k_new && t.nt > 0 && j == (L - 1) / kBlock) ? (L - 1) % kBlock : -1;
  // query heads sharing the K/V head as several pairs all read the new row from k_new/v_new;
  // the pair of the group's first query head (q row a multiple of G) stores it
  // (q rows number below 2^32: at most 4096 sequences of 2^20 query heads)
  t.store_row = -1;
  if (t.new_row >= 0 && static_cast<uint32_t>(qrow) % static_cast<uint32_t>(a.G) == 0)
    t.store_row = t.new_row;
  if (t.nt == kBlock && t.new_row < 0 && (!WIN || t.lo == 0)) {
    const int lane_off = g * G::ROW + c * 16;
#pragma unroll
    for (int i = 0; i < G::LOADS; ++i) {
      t.k[i] = load_stream(kt + lane_off + i * G::TPL * G::ROW);
      t.v[i] = load_stream(vt + lane_off + i * G::TPL * G::ROW);
    }
  } else {
    // rows past the end load the last valid row again (the same cache lines, so no extra
    // traffic; with nt = 0, row 0), rows before a window's start its first row: their scores
    // are masked to -inf, so they weigh 0
    const int64_t new_off = bkv * G::ROW + c * 16;
    const int last_row = max(t.nt, 1) - 1;
#pragma unroll
    for (int i = 0; i < G::LOADS; ++i) {
      const int row = min(WIN ? max(g + i * G::TPL, t.lo) : g + i * G::TPL, last_row);
      const bool nw = row == t.new_row;
      t.k[i] = load_stream(nw ? a.k_new + new_off : kt + row * G::ROW + c * 16);
      t.v[i] = load_stream(nw ? a.v_new + new_off : vt + row * G::ROW + c * 16);
    }
  }
}

// Append mode: store the new token's row (already in registers) into the cache.
template <int KV, int D, bool QF16, int GQ>
__device__ __forceinline__ void store_new_row(const TileRegs<KV, D, QF16, GQ> &t, int g, int c) {
  using G = Geo<KV, D>;
  if (t.store_row < 0) return;
  const int lane_off = g * G::ROW + c * 16;
#pragma unroll
  for (int i = 0; i < G::LOADS; ++i) {
    if (g + i * G::TPL == t.store_row) {
      *reinterpret_cast<uint4 *>(const_cast<char *>(t.kt) + lane_off + i * G::TPL * G::ROW) =
          t.k[i];
      *reinterpret_cast<uint4 *>(const_cast<char *>(t.vt) + lane_off + i * G::TPL * G::ROW) =
          t.v[i];
    }
  }
}

// Read every register of a tile that adds nothing (nt = 0) in an empty asm statement, so that
// no load into them stays outstanding into the fetch that next reuses them.
template <int KV, int D, bool QF16, int GQ>
__device__ __forceinline__ void touch_tile(const TileRegs<KV, D, QF16, GQ> &t) {
  using G = Geo<KV, D>;
#pragma unroll
  for (int i = 0; i < G::LOADS; ++i) {
    asm volatile("" ::"v"(t.k[i].x), "v"(t.k[i].y), "v"(t.k[i].z), "v"(t.k[i].w));
    asm volatile("" ::"v"(t.v[i].x), "v"(t.v[i].y), "v"(t.v[i].z), "v"(t.v[i].w));
  }
  if constexpr (GQ == 1) {
#pragma unroll
    for (int u = 0; u < QWords<QF16, G::EPL>::W; ++u) asm volatile("" ::"v"(t.q[0].w[u]));
  }
}

// The 16 loaded bytes of a K row as fp16 pairs (element pairs 2u, 2u + 1), exactly: fp16 as
// stored; every e4m3 code and every int8 code is an fp16 value.
template <int KV, int NP>
__device__ __forceinline__ void unpack_pairs(const uint4 &r, f16x2 *h) {
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
  if constexpr (KV == KVC_F16) {
    static_assert(NP == 4, "8 fp16 per 16 bytes");
#pragma unroll
    for (int i = 0; i < 4; ++i) h[i] = __builtin_bit_cast(f16x2, w[i]);
  } else if constexpr (KV == KVC_I8) {
    static_assert(NP == 8, "16 codes per 16 bytes");
#pragma unroll
    for (int i = 0; i < 4; ++i) i8x4_to_f16(w[i], h[2 * i], h[2 * i + 1]);
  } else {
    static_assert(NP == 8, "16 codes per 16 bytes");
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      h[2 * i] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(static_cast<int>(w[i]), 1.0f, false);
      h[2 * i + 1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(static_cast<int>(w[i]), 1.0f, true);
    }
  }
}

// Partial dot product of this lane's 16 loaded bytes of one K row with its q slice. With an fp16
// q and an fp16 or 8-bit cache, both sides are fp16 pairs and v_dot2_f32_f16 takes two products
// (exact in fp32) per instruction into the fp32 sum; otherwise the elements are widened to fp32
// and summed with FMAs.
template <int KV, bool QF16, int EPL>
__device__ __forceinline__ float dot_slice(const uint4 &kr, const QWords<QF16, EPL> &q) {
  if constexpr (QF16 && KV != KVC_F32) {
    f16x2 kh[EPL / 2];
    unpack_pairs<KV, EPL / 2>(kr, kh);
    float d = 0.f;
#pragma unroll
    for (int u = 0; u < EPL / 2; ++u)
      d = __builtin_amdgcn_fdot2(kh[u], __builtin_bit_cast(f16x2, q.w[u]), d, false);
    return d;
  } else {
    float kf[EPL], qv[EPL];
    unpack<KV>(kr, kf);
    q_floats<QF16, EPL>(q, qv);
    float d = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) d = __builtin_fmaf(kf[e], qv[e], d);
    return d;
  }
}

// ---- one tile: online-softmax update of the group state ---------------------------------
// Rows at or past nt (and below lo) get score -inf (weight 0); their V registers hold a valid
// row's data. A tile with nt = 0 adds nothing. With GQ query heads per wavefront, each head r
// keeps its own state (m[r], l[r], acc[r]) and reads the q slice qs[r]; the K and V registers
// are shared.
template <int KV, int D, bool QF16, int GQ, bool WIN>
__device__ __forceinline__ void consume_tile(const TileRegs<KV, D, QF16, GQ> &t,
                                             const QWords<QF16, Geo<KV, D>::EPL> *qs, float cl2,
                                             int g, float *m, float *l,
                                             float (*acc)[Geo<KV, D>::EPL]) {
  using G = Geo<KV, D>;
  if (t.nt <= 0) {
    touch_tile(t);
    return;
  }
  const QWords<QF16, G::EPL> *qq = GQ == 1 ? t.q : qs;
  float s[GQ][G::LOADS];
  const float sc = is_q8(KV) ? cl2 * t.ks : cl2;
#pragma unroll
  for (int i = 0; i < G::LOADS; ++i) {
    const bool ok = g + i * G::TPL < t.nt && (!WIN || g + i * G::TPL >= t.lo);
#pragma unroll
    for (int r = 0; r < GQ; ++r) {
      const float d = group_sum<G::LPT>(dot_slice<KV, QF16, G::EPL>(t.k[i], qq[r])) * sc;
      s[r][i] = ok ? d : -__builtin_inff();
    }
  }
  // The reference m moves only when a score passes it by more than kRefHeadroom (always on the
  // first tile, which starts at kFloor), and then to the tile's maximum: most tiles rescale
  // nothing. Weights stay below 2^kRefHeadroom, far inside the fp32 range.
  constexpr float kRefHeadroom = 32.f;
#pragma unroll
  for (int r = 0; r < GQ; ++r) {
    float mb = s[r][0];
#pragma unroll
    for (int i = 1; i < G::LOADS; ++i) mb = fmaxf(mb, s[r][i]);
    if (__ballot(mb > m[r] + kRefHeadroom) != 0) {
      const float mn = fmaxf(m[r], mb);
      const float alpha = __builtin_amdgcn_exp2f(m[r] - mn);
      l[r] *= alpha;
#pragma unroll
      for (int e = 0; e < G::EPL; ++e) acc[r][e] *= alpha;
      m[r] = mn;
    }
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < G::LOADS; ++i) {
      s[r][i] = __builtin_amdgcn_exp2f(s[r][i] - m[r]);  // now the weight p
      psum += s[r][i];
    }
    l[r] += psum;
  }
#pragma unroll
  for (int i = 0; i < G::LOADS; ++i) {
    float vf[G::EPL];
    unpack<KV>(t.v[i], vf);
#pragma unroll
    for (int r = 0; r < GQ; ++r) {
      const float pi = is_q8(KV) ? s[r][i] * t.vs : s[r][i];
#pragma unroll
      for (int e = 0; e < G::EPL; ++e) acc[r][e] = __builtin_fmaf(pi, vf[e], acc[r][e]);
    }
  }
}

// ---- the wavefront's chunk: segments and the tile pipeline --------------------------------
// A segment is the part of one (sequence, head) pair that lies in the chunk: tiles j0 .. j0+n-1.
struct Seg {
  int32_t b, h, j0, n, L;  // h: the pair index in [0, Hp); j0: logical block of the first tile
  int32_t ph0, ph1;  // paged: block ids of the segment's first two tiles (-1 past the end)
  bool cut_start, cut_end;
};

// Workgroup x of a launch of n runs on XCD x % 8 (round-robin dispatch). Logical workgroup
// xcd_major(x, n) numbers the workgroups so that each XCD holds a contiguous range of them, the
// ranges as even as n allows (a bijection of [0, n)).
__device__ __forceinline__ int32_t xcd_major(int32_t x, int32_t n) {
  const int32_t xcd = x % 8, q = n / 8, rem = n % 8;
  return xcd * q + min(xcd, rem) + x / 8;
}

// The order of the work list. Sequence-major (contiguous caches): sequence b's pairs in turn,
// so tile f is tile f - Hp pre[b] - h nb of pair h of the sequence b with Hp pre[b] <= f.
// Pair-major (paged pools): pair h of every sequence in turn, then pair h + 1, so tile f is tile
// f - h T - pre[b] of pair h of sequence b, T = pre[B] tiles per pair row. Sequences of a paged
// pool can share blocks (the candidates of parallel sampling share their prompt's): with the
// list pair-major and each XCD taking a contiguous range of it (xcd_major), the candidates'
// reads of one shared block come from one XCD and meet in its L2. In both orders a pair's tiles
// are consecutive, so a cursor moves from pair to pair by adding the pair's tile count.
struct ChunkStart {
  int32_t b, h, base;  // the pair holding the chunk's first tile, and the pair's first tile
};

// The pair a chunk cursor is in: its indices, first tile, tile count and sequence length (read
// from LDS once per pair, not once per segment).
struct SeqCur {
  int32_t b, h, base, nb, L;
  int32_t jb;  // first logical block the sequence attends (rolling window; else 0)
};

template <bool WIN>
__device__ __forceinline__ void load_seq(const DecodeArgs &a, const int32_t *pre,
                                         const int32_t *len, int32_t b, int32_t h, int32_t base,
                                         SeqCur &q) {
  q.b = b;
  q.h = h;
  q.base = base;
  q.nb = sread(pre + b + 1) - sread(pre + b);
  q.L = sread(len + b);
  q.jb = window_block<WIN>(q.L, a.window);
}

// Next segment of the chunk starting at tile f (the cursor only moves forward, pair by pair in
// the list's order). Returns false at the end of the chunk.
template <bool WIN>
__device__ __forceinline__ bool next_seg(const DecodeArgs &a, const int32_t *pre,
                                         const int32_t *len, int32_t &f, int32_t f1, SeqCur &q,
                                         Seg &s) {
  if (f >= f1) return false;
  while (f >= q.base + q.nb) {  // f < total: ends
    int32_t b = q.b, h = q.h;
    if (a.pair_major) {
      const bool wrap = b + 1 == a.B;
      b = wrap ? 0 : b + 1;
      h = wrap ? h + 1 : h;
    } else {
      const bool wrap = h + 1 == a.Hp;
      h = wrap ? 0 : h + 1;
      b = wrap ? b + 1 : b;
    }
    load_seq<WIN>(a, pre, len, b, h, q.base + q.nb, q);
  }
  s.b = q.b;
  s.h = q.h;
  s.j0 = f - q.base;
  const int32_t seg_end = q.base + q.nb;
  const int32_t e = min(f1, seg_end);
  s.n = e - f;
  s.cut_start = s.j0 > 0;
  s.cut_end = e < seg_end;
  s.L = q.L;
  if constexpr (WIN) s.j0 += q.jb;  // from here on j0 is the logical block of the first tile
  f = e;
  return true;
}

// Block id of tile j of sequence b (scalar load).
__device__ __forceinline__ int32_t block_id(const DecodeArgs &a, int32_t b, int32_t j) {
  return sload(a.tables + static_cast<int64_t>(b) * a.mbps + j);
}

template <bool PAGED>
__device__ __forceinline__ void seg_ids(const DecodeArgs &a, Seg &s) {
  if constexpr (PAGED) {
    s.ph0 = block_id(a, s.b, s.j0);
    s.ph1 = s.n > 1 ? block_id(a, s.b, s.j0 + 1) : -1;
  }
}


// One level of the combination of lane groups' states (running max m, sum l, output acc): each
// lane merges its state with the one OFF lanes away. The merge is symmetric in the two states,
// so after the levels for OFF = LPT, 2*LPT, ..., 32 lane group 0 holds the whole segment's.
template <int OFF, int EPL>
__device__ __forceinline__ void merge_lanes(float &m, float &l, float *acc) {
  float ma, mb, la, lb;
  lane_pair<OFF>(m, ma, mb);
  lane_pair<OFF>(l, la, lb);
  const float M = fmaxf(ma, mb);
  const float fa = __builtin_amdgcn_exp2f(ma - M);
  const float fb = __builtin_amdgcn_exp2f(mb - M);
  l = la * fa + lb * fb;
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    float xa, xb;
    lane_pair<OFF>(acc[e], xa, xb);
    acc[e] = xa * fa + xb * fb;
  }
  m = M;
}

// LDS of a pass-1 workgroup: pre[B+1], len[B], wsum[kWgWaves], then (16-byte aligned) the
// stages of its wavefronts, then (workgroup combine) their edge slots and the slots'
// descriptions, then (matrix cores) one fp16 V tile per wavefront.
__host__ __device__ inline int32_t stage_offset(int32_t B) { return (2 * B + 1 + kWgWaves + 3) & ~3; }

struct LdsPlan {
  size_t edge, einfo, vbuf, total;  // byte offsets from the start of LDS, and the total
};

__host__ __device__ inline LdsPlan lds_plan(int32_t B, int32_t D, int32_t stage_rows, int32_t gq,
                                            bool wg_combine, bool mfma) {
  LdsPlan p;
  p.edge = (static_cast<size_t>(stage_offset(B)) +
            static_cast<size_t>(kWgWaves) * stage_rows * (D + 4)) * sizeof(float);
  p.einfo = p.edge + (wg_combine ? static_cast<size_t>(kWgWaves) * 2 * gq * (D + 4) * sizeof(float)
                                 : 0);
  p.vbuf = p.einfo + (wg_combine ? static_cast<size_t>(kWgWaves) * 4 * sizeof(int32_t) : 0);
  p.total = p.vbuf + (mfma ? static_cast<size_t>(kWgWaves) * kBlock * D * 2 : 0);
  return p;
}

// Finished segments wait in LDS until the wavefront's loads are done (or the stage is full), so
// that no global store sits between a tile's loads and the wait for them: a wait for loads on
// this GPU also waits for every store issued before it. A row entry is D+4 floats: the combined
// unnormalised output, then m, l and the destination (int bits: >= 0 the output row b*Hq+hq;
// < 0 the record row -1-r).
struct Stage {
  float *base;  // this wavefront's entries (DecodeArgs::stage_rows of them)
  int32_t n;    // entries in use
  // workgroup combine: the wavefront's two edge slots (0: the segment cut at its chunk's start,
  // 1: the one cut at its end; GQ entries each) and their descriptions {pair, flags} (flags bit
  // 0: holds an entry, bit 1: cut at the start, bit 2: cut at the end); null otherwise
  float *edge;
  int32_t *einfo;
};

// Where a finished segment's entries go: an edge slot when the workgroup combines cut pairs and
// the segment was cut, else the stage (flushed first if its GQ entries do not fit).
template <int D>
__device__ __forceinline__ float *segment_entries(const DecodeArgs &a, const Seg &sg, int32_t gq,
                                                  int32_t stage_rows, Stage &st, bool &to_edge);

// Store the staged entries: output rows normalised by 1/l (fp16 rounded to nearest even, or
// fp32), records copied with their m and l. Every lane takes columns lane, lane+64, ...
template <int D>
__device__ __forceinline__ void flush_stage(const DecodeArgs &a, Stage &st) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int lane = threadIdx.x & (kWave - 1);
  for (int32_t k = 0; k < st.n; ++k) {
    const float *e = st.base + k * (D + 4);
    const int32_t dest = __float_as_int(e[D + 2]);
    if (dest >= 0) {
      const float l = e[D + 1];
      const float inv = l > 0.f ? 1.0f / l : 0.f;
#pragma unroll
      for (int d = lane; d < D; d += kWave)
        store_elem(a.out, static_cast<int64_t>(dest) * D + d, e[d] * inv, a.out_f16);
    } else {
      float *r = a.ws_rec + static_cast<int64_t>(-1 - dest) * (D + 4);
      for (int d = lane; d < D + 2; d += kWave) r[d] = e[d];
    }
  }
  st.n = 0;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int D>
__device__ __forceinline__ float *segment_entries(const DecodeArgs &a, const Seg &sg, int32_t gq,
                                                  int32_t stage_rows, Stage &st, bool &to_edge) {
  to_edge = st.edge != nullptr && (sg.cut_start || sg.cut_end);
  if (to_edge) {
    const int slot = sg.cut_start ? 0 : 1;
    if ((threadIdx.x & (kWave - 1)) == 0) {
      st.einfo[2 * slot] = sg.b * a.Hp + sg.h;
      st.einfo[2 * slot + 1] = 1 | (sg.cut_start ? 2 : 0) | (sg.cut_end ? 4 : 0);
    }
    return st.edge + slot * gq * (D + 4);
  }
  if (st.n + gq > stage_rows) flush_stage<D>(a, st);
  return st.base + st.n * (D + 4);
}

// Finish a segment: for each of its GQ query heads combine the TPL lane groups, then stage
// either the output row (the whole pair was in this chunk) or a record (slot 0 if the pair
// began before the chunk, else 1; the record of head r is row (2w+slot)*GQ + r), or, when the
// workgroup combines cut pairs, put a cut segment's entries in its edge slot.
template <int KV, int D, int GQ>
__device__ __forceinline__ void finish_seg(const DecodeArgs &a, const Seg &s, int32_t w, int g,
                                           int c, float *m, float *l,
                                           float (*acc)[Geo<KV, D>::EPL], Stage &st) {
  using G = Geo<KV, D>;
  bool to_edge;
  float *const e0 = segment_entries<D>(a, s, GQ, kStageRows, st, to_edge);
  const bool whole = !s.cut_start && !s.cut_end;
  const int32_t out0 = s.b * a.Hq + s.h * GQ;
  const int32_t rec0 = (w * 2 + (s.cut_start ? 0 : 1)) * GQ;
#pragma unroll
  for (int r = 0; r < GQ; ++r) {
    if constexpr (G::LPT <= 4) merge_lanes<4, G::EPL>(m[r], l[r], acc[r]);
    if constexpr (G::LPT <= 8) merge_lanes<8, G::EPL>(m[r], l[r], acc[r]);
    if constexpr (G::LPT <= 16) merge_lanes<16, G::EPL>(m[r], l[r], acc[r]);
    merge_lanes<32, G::EPL>(m[r], l[r], acc[r]);
    const int32_t dest = whole ? out0 + r : -1 - (rec0 + r);
    float *e = e0 + r * (D + 4);
    if (g == 0) {
#pragma unroll
      for (int k = 0; k < G::EPL; ++k) e[c * G::EPL + k] = acc[r][k];
      if (c == 0) {
        e[D] = m[r];
        e[D + 1] = l[r];
        e[D + 2] = __int_as_float(dest);
      }
    }
  }
  if (!to_edge) st.n += GQ;
}

// ---- pass-1 cores ---------------------------------------------------------------------------
// A core is how one wavefront loads a 16-position tile of one K/V head and folds it into the
// softmax state of the query heads it serves. run_chunk below drives a core over a chunk.
//   VecCore:  vector ALU; one query head per wavefront (multi-head attention), or two heads of a
//             group that share the tile's K/V registers.
//   MfmaCore: matrix cores; up to 16 query heads of a group against one K/V head.

// Vector core: the tile code above, one (or two) query heads per wavefront.
template <bool PAGED, int KV, int D, bool QF16, int GQ, bool WIN>
struct VecCore {
  using G = Geo<KV, D>;
  using Tile = TileRegs<KV, D, QF16, GQ>;
  static constexpr int kD = D;
  static constexpr bool kWin = WIN;
  struct State {
    QWords<QF16, G::EPL> qs[GQ];  // GQ > 1: the segment's q slices
    float m[GQ], l[GQ];
    float acc[GQ][G::EPL];
  };
  int g, c;  // the lane's row within a wave-wide load, and its 16-byte column

  __device__ explicit VecCore(int lane) : g(lane / G::LPT), c(lane % G::LPT) {}
  __device__ int32_t gq(const DecodeArgs &) const { return GQ; }

  __device__ void fetch(const DecodeArgs &a, Tile &t, int64_t bkv, int32_t hkv, int64_t qrow,
                        int32_t j, int32_t phys, int32_t L, bool live) const {
    fetch_tile<PAGED, KV, D, QF16, GQ, WIN>(a, t, bkv, hkv, qrow, j, phys, L, live, g, c);
  }
  // A segment becomes current: its q slices (GQ > 1) and a fresh softmax state.
  __device__ void begin(const DecodeArgs &a, int64_t qrow, State &s) const {
    if constexpr (GQ > 1) {
#pragma unroll
      for (int r = 0; r < GQ; ++r)
        load_q_words<QF16, G::EPL>(a.q, (qrow + r) * D + c * G::EPL, s.qs[r]);
    }
#pragma unroll
    for (int r = 0; r < GQ; ++r) {
      s.m[r] = kFloor;
      s.l[r] = 0.f;
#pragma unroll
      for (int e = 0; e < G::EPL; ++e) s.acc[r][e] = 0.f;
    }
  }
  __device__ void consume(const DecodeArgs &a, const Tile &t, State &s) const {
    consume_tile<KV, D, QF16, GQ, WIN>(t, s.qs, a.cl2, g, s.m, s.l, s.acc);
    store_new_row<KV, D, QF16, GQ>(t, g, c);
  }
  __device__ void finish(const DecodeArgs &a, const Seg &sg, int32_t w, State &s,
                         Stage &st) const {
    finish_seg<KV, D, GQ>(a, sg, w, g, c, s.m, s.l, s.acc, st);
  }
};

// Matrix-core core for grouped queries: the GQ (<= 16) query heads of a pair share every K/V
// tile, so a tile is a 16-position x D block against a 16-column block of queries. Lanes are
// (g, j) = (lane / 16, lane % 16).
//   Scores: S^T = K . Q^T with v_mfma_f32_16x16x32_f16 (D/32 of them). Lane (g, j) holds K row
//     j and q of head j (heads past GQ repeat the last one; their columns are never stored), 8
//     dims per MFMA, the same dims in both. The result gives lane (g, j) the scores of positions
//     4g..4g+3 for head j.
//   Softmax: head j's weights are exp2(score - reference), the reference shared by the four
//     lane groups. It is moved (and the output and sums rescaled) only when a tile's maximum
//     passes it by more than a fixed headroom, so a tile normally costs no rescale; the weights
//     stay below 2^15. Each lane keeps the partial sum of its own positions' weights.
//   Output: O^T = V^T . P^T with v_mfma_f32_16x16x16_f16 per 16 output dims. The B operand is
//     the weights exactly where the score MFMA left them (positions 4g..4g+3 of head j). The
//     weights enter as two fp16 terms, p = hi + lo with hi = fp16(p) and lo = fp16(p - hi), so
//     about 22 bits of each weight reach the fp32 accumulator. A needs V transposed (four
//     positions of one dim per lane): the tile goes through LDS. It is loaded in the
//     wave-contiguous layout, written as fp16 rows with 16-byte columns swizzled by row, and
//     read back with one transposing read (ds_read_b64_tr_b16) per 16 dims; the swizzle puts
//     the rows of a read on distinct banks. Lane (g, j) accumulates dims 16*dc + 4g .. +3 of
//     head j.
//   8-bit caches: e4m3 codes convert exactly to fp16 (v_cvt_scalef32_pk_f16_fp8 with scale 1),
//     int8 codes too (through a biased fp16 exponent, i8x8_to_f16). The K block
//     scale multiplies the scores. O is held in units of a reference V scale; a tile's weights
//     are multiplied by its block's scale over the reference (kept within [1/16, 16], else the
//     reference moves to this block's scale and O is rescaled).
template <bool PAGED, int KV, int D, bool WIN, bool APPEND>
struct MfmaCore {
  static_assert(KV == KVC_F16 || is_q8(KV), "fp16 or 8-bit cache");
  static_assert(!APPEND || (KV == KVC_F16 && !WIN), "append mode: fp16 cache, no window");
  using G = Geo<KV, D>;            // wave-contiguous geometry (V loads)
  static constexpr int kD = D;
  static constexpr bool kWin = WIN;
  static constexpr int KL = G::ROW / 64;  // K loads per lane per tile (16 bytes each)
  static constexpr int NQK = D / 32;      // score MFMAs per tile
  static constexpr int NDC = D / 16;      // 16-dim output blocks
  static constexpr int kVbufBytes = kBlock * D * 2;
  // Weight headroom (log2 units): weights are at most 2^kHi, times kRat for 8-bit caches, below the
  // fp16 maximum; a fresh reference gives the tile's top weight 2^kHead.
  static constexpr float kHead = is_q8(KV) ? 3.f : 7.f;
  static constexpr float kHi = is_q8(KV) ? 11.f : 15.f;
  static constexpr float kRat = 16.f;
  struct Tile {
    uint4 k[KL];
    uint4 v[G::LOADS];
    int32_t nt;
    int32_t lo;  // rolling window: rows below lo lie before the window
    float ks, vs;
    // append mode (APPEND instances), as in TileRegs: the new token's row, read from
    // k_new/v_new, and the row this wavefront stores into the cache at kt/vt (-1: none)
    int32_t new_row, store_row;
    const char *kt;
    const char *vt;
  };
  struct State {
    uint4 q[NQK];  // q operand, 8 fp16 dims per score MFMA
    f32x4 o[NDC];
    float m, l, vref;
  };
  int g, j;        // MFMA role
  int gv, cv;      // wave-contiguous role: row gv + TPL*i, 16-byte column cv
  _Float16 *vbuf;  // this wavefront's LDS tile, [16][D] fp16

  __device__ MfmaCore(int lane, _Float16 *buf)
      : g(lane >> 4), j(lane & 15), gv(lane / G::LPT), cv(lane % G::LPT), vbuf(buf) {}
  __device__ int32_t gq(const DecodeArgs &a) const { return a.gq; }

  // LDS column (8 fp16) of 16-byte column c of row t. The transposing V reads take, per 32
  // lanes, 2 adjacent columns (from an even one) of 8 consecutive rows, 8 bytes a lane: with
  // 256-byte rows (D = 128) the row's low three bits move the column's upper three; with 128-byte
  // rows (D = 64, two rows per 256-byte bank line) bits 1-2 of the row move them. The 16-byte
  // row writes stay on distinct banks too.
  static __device__ __forceinline__ int swz(int t, int c) {
    return D == 128 ? c ^ (2 * (t & 7)) : c ^ (2 * ((t >> 1) & 3));
  }

  __device__ void fetch(const DecodeArgs &a, Tile &t, int64_t bkv, int32_t hkv, int64_t qrow,
                        int32_t jt, int32_t phys, int32_t L, bool live) const {
    const char *kt;
    const char *vt;
    bool valid = live;
    if constexpr (PAGED) {
      valid = valid && static_cast<uint32_t>(phys) < static_cast<uint32_t>(a.num_blocks);
      const int32_t sp = valid ? phys : 0;
      const int64_t toff = (static_cast<int64_t>(sp) * a.H + hkv) * G::TILE;
      kt = a.k + toff;
      vt = a.v + toff;
      if constexpr (is_q8(KV)) {
        t.ks = valid ? a.k_scale[sp] : 0.f;
        t.vs = valid ? a.v_scale[sp] : 0.f;
      }
    } else {
      const int64_t toff = (bkv * a.seq_stride + static_cast<int64_t>(kBlock) * (valid ? jt : 0)) *
                           G::ROW;
      kt = a.k + toff;
      vt = a.v + toff;
    }
    t.nt = valid ? min(kBlock, L - kBlock * jt) : 0;
    t.lo = WIN ? min(max(max(0, L - a.window) - kBlock * jt, 0), kBlock) : 0;
    // rows past the end read the last valid row (the same lines), rows before a window's start
    // its first row: their weights are 0, and their V values are finite, so 0 * v stays 0
    const int last = max(t.nt, 1) - 1;
    auto row_of = [&](int r) { return min(WIN ? max(r, t.lo) : r, last); };
    if constexpr (APPEND) {
      // the tile of the new token (its last row, so rows past the end repeat it): lanes of that
      // row load it from k_new/v_new; the group's first pair stores it when the tile is consumed
      t.kt = kt;
      t.vt = vt;
      const bool has_new = t.nt > 0 && jt == (L - 1) / kBlock;  // wave-uniform
      t.new_row = has_new ? last : -1;
      t.store_row = -1;
      if (has_new && static_cast<uint32_t>(qrow) % static_cast<uint32_t>(a.G) == 0)
        t.store_row = last;
      const int64_t new_off = bkv * G::ROW;
      const int rk = row_of(j);
      const char *kr = rk == t.new_row ? a.k_new + new_off + g * 16 : kt + rk * G::ROW + g * 16;
#pragma unroll
      for (int c = 0; c < KL; ++c) t.k[c] = load_stream(kr + c * 64);
#pragma unroll
      for (int i = 0; i < G::LOADS; ++i) {
        const int r = row_of(gv + i * G::TPL);
        t.v[i] = load_stream(r == t.new_row ? a.v_new + new_off + cv * 16
                                            : vt + r * G::ROW + cv * 16);
      }
      return;
    }
    const char *kr = kt + row_of(j) * G::ROW + g * 16;
#pragma unroll
    for (int c = 0; c < KL; ++c) t.k[c] = load_stream(kr + c * 64);
#pragma unroll
    for (int i = 0; i < G::LOADS; ++i)
      t.v[i] = load_stream(vt + row_of(gv + i * G::TPL) * G::ROW + cv * 16);
  }

  // Append mode: the lanes holding the new row store it into the cache (K: lanes of MFMA row
  // store_row, 64 bytes apart; V: the wave-contiguous lanes of that row).
  __device__ void store_new(const Tile &t) const {
    if constexpr (APPEND) {
      if (t.store_row < 0) return;
      if (j == t.store_row) {
#pragma unroll
        for (int c = 0; c < KL; ++c)
          *reinterpret_cast<uint4 *>(const_cast<char *>(t.kt) + t.store_row * G::ROW + g * 16 +
                                     c * 64) = t.k[c];
      }
#pragma unroll
      for (int i = 0; i < G::LOADS; ++i) {
        if (gv + i * G::TPL == t.store_row)
          *reinterpret_cast<uint4 *>(const_cast<char *>(t.vt) + t.store_row * G::ROW +
                                     cv * 16) = t.v[i];
      }
    }
  }

  // q operand of head j of the pair: 16-byte chunk of the fp16 q row for score MFMA n (the dims
  // K load n / 2 half n % 2 covers for 8-bit caches, K load n for fp16)
  __device__ void begin(const DecodeArgs &a, int64_t qrow, State &s) const {
    const char *qr = static_cast<const char *>(a.q) + (qrow + min(j, a.gq - 1)) * (D * 2);
#pragma unroll
    for (int n = 0; n < NQK; ++n) {
      const int chunk = KV == KVC_F16 ? g + 4 * n : 2 * (g + 4 * (n >> 1)) + (n & 1);
      s.q[n] = *reinterpret_cast<const uint4 *>(qr + chunk * 16);
    }
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) s.o[dc] = f32x4{0.f, 0.f, 0.f, 0.f};
    s.m = kFloor;
    s.l = 0.f;
    s.vref = 1.f;
  }

  // 8 codes of the cache's 8-bit format as fp16, exactly
  static __device__ __forceinline__ f16x8 q8x8_to_f16(uint32_t w0, uint32_t w1) {
    if constexpr (KV == KVC_I8) return i8x8_to_f16(w0, w1);
    return fp8x8_to_f16(w0, w1);
  }

  __device__ void touch(const Tile &t) const {
#pragma unroll
    for (int c = 0; c < KL; ++c)
      asm volatile("" ::"v"(t.k[c].x), "v"(t.k[c].y), "v"(t.k[c].z), "v"(t.k[c].w));
#pragma unroll
    for (int i = 0; i < G::LOADS; ++i)
      asm volatile("" ::"v"(t.v[i].x), "v"(t.v[i].y), "v"(t.v[i].z), "v"(t.v[i].w));
  }

  __device__ void consume(const DecodeArgs &a, const Tile &t, State &s) const {
    if (t.nt <= 0) {
      touch(t);
      return;
    }
    // V rows into LDS as fp16
#pragma unroll
    for (int i = 0; i < G::LOADS; ++i) {
      const int row = gv + i * G::TPL;
      if constexpr (KV == KVC_F16) {
        *reinterpret_cast<uint4 *>(vbuf + row * D + swz(row, cv) * 8) = t.v[i];
      } else {
        *reinterpret_cast<f16x8 *>(vbuf + row * D + swz(row, 2 * cv) * 8) =
            q8x8_to_f16(t.v[i].x, t.v[i].y);
        *reinterpret_cast<f16x8 *>(vbuf + row * D + swz(row, 2 * cv + 1) * 8) =
            q8x8_to_f16(t.v[i].z, t.v[i].w);
      }
    }
    store_new(t);
    // scores of positions 4g..4g+3 for head j
    f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int n = 0; n < NQK; ++n) {
      f16x8 ka;
      if constexpr (KV == KVC_F16) {
        ka = as_f16x8(t.k[n]);
      } else {
        const uint4 &w = t.k[n >> 1];
        ka = (n & 1) ? q8x8_to_f16(w.z, w.w) : q8x8_to_f16(w.x, w.y);
      }
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, as_f16x8(s.q[n]), sacc, 0, 0, 0);
    }
    const float sc = is_q8(KV) ? a.cl2 * t.ks : a.cl2;
    float x[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      x[e] = 4 * g + e < t.nt && (!WIN || 4 * g + e >= t.lo) ? sacc[e] * sc : -__builtin_inff();
    float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    {
      float u, v;
      lane_pair<16>(mx, u, v);
      mx = fmaxf(u, v);
      lane_pair<32>(mx, u, v);
      mx = fmaxf(u, v);
    }
    // The reference moves only when a score passes it by more than kHi (first tile included,
    // since it starts at kFloor); then it is set kHead below the tile's maximum. 8-bit: the ratio
    // of this block's V scale to the reference scale must also stay within [1/kRat, kRat].
    float ratio = 1.f;
    bool rebase = false;
    float vsn = 1.f;
    if constexpr (is_q8(KV)) {
      // an all-zero block has scale 0 and zero codes: any scale represents it
      vsn = t.vs != 0.f ? t.vs : 1.f;
      ratio = vsn / s.vref;
      rebase = !(ratio <= kRat && ratio >= 1.f / kRat);
    }
    const bool up = mx > s.m + kHi;
    if (__ballot(up) != 0 || rebase) {
      const float mnew = up ? mx - kHead : s.m;
      float f = __builtin_amdgcn_exp2f(s.m - mnew);
      s.l *= f;
      if constexpr (is_q8(KV)) {
        f *= s.vref / vsn;
        s.vref = vsn;
        ratio = 1.f;
      }
#pragma unroll
      for (int dc = 0; dc < NDC; ++dc) s.o[dc] *= f;
      s.m = mnew;
    }
    float p[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      p[e] = __builtin_amdgcn_exp2f(x[e] - s.m);
      s.l += p[e];
    }
    f16x4 ph, pl;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float pv = is_q8(KV) ? p[e] * ratio : p[e];
      ph[e] = static_cast<_Float16>(pv);
      pl[e] = static_cast<_Float16>(pv - static_cast<float>(ph[e]));
    }
    wave_lds_sync();
    // V^T: dims 16dc + j of positions 4g..4g+3, one gfx950 transposing read per 16 dims (in
    // each 16-lane group, lane 4i + e receives element e of the 8 bytes that lanes i, i + 4,
    // i + 8 and i + 12 address): lane s of group g addresses row 4g + s/4, dims
    // 16dc + 4(s%4) .. + 3
    const int vrow = 4 * g + (j >> 2);
    const char *vr = reinterpret_cast<const char *>(vbuf + vrow * D) + (j & 1) * 8;
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) {
      const char *vp = vr + swz(vrow, 2 * dc + ((j >> 1) & 1)) * 16;
      const f16x4 va = __builtin_bit_cast(
          f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                     (__attribute__((address_space(3))) i16x4 *)(vp)));
      s.o[dc] = __builtin_amdgcn_mfma_f32_16x16x16f16(va, ph, s.o[dc], 0, 0, 0);
      s.o[dc] = __builtin_amdgcn_mfma_f32_16x16x16f16(va, pl, s.o[dc], 0, 0, 0);
    }
    wave_lds_sync();
  }

  // Finish a segment: head j's weight sum over the four lane groups, then stage its output row
  // or record (as finish_seg does; the record of head r is row (2w + slot) * gq + r).
  __device__ void finish(const DecodeArgs &a, const Seg &sg, int32_t w, State &s,
                         Stage &st) const {
    float u, v;
    lane_pair<16>(s.l, u, v);
    float l = u + v;
    lane_pair<32>(l, u, v);
    l = u + v;
    const int32_t GQ = a.gq;
    bool to_edge;
    float *const e0 = segment_entries<D>(a, sg, GQ, a.stage_rows, st, to_edge);
    const bool whole = !sg.cut_start && !sg.cut_end;
    const int32_t out0 = sg.b * a.Hq + sg.h * GQ;
    const int32_t rec0 = (w * 2 + (sg.cut_start ? 0 : 1)) * GQ;
    if (j < GQ) {
      float *e = e0 + j * (D + 4);
      const float vr = is_q8(KV) ? s.vref : 1.f;
#pragma unroll
      for (int dc = 0; dc < NDC; ++dc)
        *reinterpret_cast<f32x4 *>(e + 16 * dc + 4 * g) = s.o[dc] * vr;
      if (g == 0) {
        e[D] = s.m;
        e[D + 1] = l;
        e[D + 2] = __int_as_float(whole ? out0 + j : -1 - (rec0 + j));
      }
    }
    if (!to_edge) st.n += GQ;
  }
};

// Walk the chunk [f0, f1) tile by tile as one pipeline: while tile t is consumed, tile t+1 is in
// flight, also across segment boundaries. Every step issues one fetch of the same shape (after
// the chunk's last tile, a stand-in that is not consumed). Paged block ids come through the
// scalar cache one tile ahead of their use (a segment's first two when the segment is found).
// A segment's per-segment registers (q of its heads when a wavefront serves several) are loaded
// when it becomes current, after the loads of its first tile.
template <bool PAGED, class Core>
__device__ __forceinline__ void run_chunk(const DecodeArgs &a, const int32_t *pre,
                                          const int32_t *len, int32_t f0, int32_t f1,
                                          ChunkStart cs, int32_t w, Stage &st, const Core &core,
                                          bool flush_at_end) {
  using Tile = typename Core::Tile;
  const int32_t GQ = core.gq(a);
  int32_t f = f0;
  constexpr bool WIN = Core::kWin;
  SeqCur sq;
  load_seq<WIN>(a, pre, len, cs.b, cs.h, cs.base, sq);

  Seg cur, nxt;
  next_seg<WIN>(a, pre, len, f, f1, sq, cur);  // f0 < f1, so there is a first segment
  seg_ids<PAGED>(a, cur);
  bool has_nxt = next_seg<WIN>(a, pre, len, f, f1, sq, nxt);
  if (has_nxt) seg_ids<PAGED>(a, nxt);

  // K/V head and first q row of a pair h of sequence b
  auto bkv_of = [&](int32_t b, int32_t h) -> int64_t {
    return static_cast<int64_t>(b) * a.H + h / a.nsub;
  };
  auto qrow_of = [&](int32_t b, int32_t h) -> int64_t {
    return static_cast<int64_t>(b) * a.Hq + static_cast<int64_t>(h) * GQ;
  };
  typename Core::State s;

  int32_t i = 0;        // index, within the current segment, of the tile being consumed
  int32_t ph_next = 0;  // paged: block id of tile i+1 of the current segment (-1 past its end)
  if constexpr (PAGED) ph_next = cur.ph1;
  // one pipeline step: issue the next fetch into `nb`, consume `cb`; false when the chunk is done
  auto step = [&](Tile &cb, Tile &nb) -> bool {
    const bool last = i + 1 == cur.n;
    const bool to_nxt = last && has_nxt;
    {
      // one load site (scalar selects pick the tile): the next tile of this segment, the first
      // of the next one, or after the chunk's end a stand-in
      const int32_t ph = to_nxt ? nxt.ph0 : ph_next;
      const int32_t b = to_nxt ? nxt.b : cur.b;
      const int32_t h = to_nxt ? nxt.h : cur.h;
      const int32_t j = to_nxt ? nxt.j0 : cur.j0 + i + 1;
      const int32_t L = to_nxt ? nxt.L : cur.L;
      core.fetch(a, nb, bkv_of(b, h), h / a.nsub, qrow_of(b, h), j, ph, L, !last || has_nxt);
    }
    if constexpr (PAGED) ph_next = i + 2 < cur.n ? block_id(a, cur.b, cur.j0 + i + 2) : -1;
    core.consume(a, cb, s);
    if (!last) {
      ++i;
      return true;
    }
    core.finish(a, cur, w, s, st);
    if (!has_nxt) return false;
    cur = nxt;
    core.begin(a, qrow_of(cur.b, cur.h), s);
    i = 0;
    if constexpr (PAGED) ph_next = cur.ph1;
    has_nxt = next_seg<WIN>(a, pre, len, f, f1, sq, nxt);
    if (has_nxt) seg_ids<PAGED>(a, nxt);
    return true;
  };

  Tile ta, tb;
  core.fetch(a, ta, bkv_of(cur.b, cur.h), cur.h / a.nsub, qrow_of(cur.b, cur.h), cur.j0,
             PAGED ? cur.ph0 : 0, cur.L, true);
  core.begin(a, qrow_of(cur.b, cur.h), s);
  for (;;) {
    if (!step(ta, tb)) break;
    if (!step(tb, ta)) break;
  }
  if (flush_at_end) flush_stage<Core::kD>(a, st);
}

// The body of both pass-1 kernels: block prefix, header, the wavefront's chunk, the walk. LDS:
// pre, len, wsum, then a.stage_rows staged rows per wavefront, then (matrix cores) one fp16 V
// tile per wavefront.
template <bool PAGED, class Core, int D>
__device__ __forceinline__ Stage partial_setup(const DecodeArgs &a, int32_t *smem, int32_t gq,
                                               int32_t &f0_out, int32_t &f1_out,
                                               ChunkStart &cs_out, int32_t &w_out) {
  int32_t *pre = smem;
  int32_t *len = smem + a.B + 1;
  int32_t *wsum = len + a.B;
  Stage st;
  st.base = reinterpret_cast<float *>(smem + stage_offset(a.B)) +
            (threadIdx.x >> 6) * a.stage_rows * (D + 4);
  st.n = 0;
  st.edge = nullptr;
  st.einfo = nullptr;
  if (a.wg_combine) {
    const LdsPlan lp = lds_plan(a.B, D, a.stage_rows, gq, true, false);
    char *lds = reinterpret_cast<char *>(smem);
    const int wave = threadIdx.x >> 6;
    st.edge = reinterpret_cast<float *>(lds + lp.edge) + wave * 2 * gq * (D + 4);
    st.einfo = reinterpret_cast<int32_t *>(lds + lp.einfo) + wave * 4;
    if ((threadIdx.x & (kWave - 1)) == 0) {
      st.einfo[1] = 0;
      st.einfo[3] = 0;
    }
  }
  if (a.pair_mode) {
    // workgroup x takes pair x = (b, h) whole; its tiles are numbered from 0 at the start of
    // sequence b (pre[b] = 0, pre[b+1] = tiles per pair) and cut into one chunk per wavefront
    const int32_t x = static_cast<int32_t>(blockIdx.x);
    const int32_t b = x / a.Hp;
    const int32_t h = x - b * a.Hp;
    const int32_t L = min(max(a.lens[b], 0), a.cap);
    const int32_t nb = (L + kBlock - 1) / kBlock - window_block<Core::kWin>(L, a.window);
    if (threadIdx.x == 0) {
      pre[b] = 0;
      pre[b + 1] = nb;
      len[b] = L;
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) {
      a.ws_hdr[0] = 0;
      a.ws_hdr[1] = a.B;
      a.ws_hdr[2] = a.Hp;
      a.ws_hdr[3] = D;
      a.ws_hdr[4] = gq;
      a.ws_hdr[5] = 1;  // every output row is written by pass 1: the merge has nothing to do
      a.ws_hdr[6] = a.pair_major;
    }
    __syncthreads();
    const int32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int32_t c = (nb + kWgWaves - 1) / kWgWaves;
    w_out = x * kWgWaves + wave;
    f0_out = h * nb + min(wave * c, nb);
    f1_out = h * nb + min(wave * c + c, nb);
    cs_out = ChunkStart{b, h, h * nb};  // the workgroup's list: pair h of sequence b alone
    return st;
  }
  block_prefix<Core::kWin>(a.lens, a.B, a.cap, a.window, pre, len, wsum);

  const int32_t total = a.Hp * pre[a.B];
  const int32_t C = max(a.cmin, (total + a.P - 1) / a.P);
  if (blockIdx.x == 0) {
    for (int i = threadIdx.x; i <= a.B; i += kWgThreads) a.ws_pre[i] = pre[i];
    if (threadIdx.x == 0) {
      // the merge's parts: wavefronts, or whole workgroups when they combine their own cuts
      a.ws_hdr[0] = a.wg_combine ? C * kWgWaves : C;
      a.ws_hdr[1] = a.B;
      a.ws_hdr[2] = a.Hp;
      a.ws_hdr[3] = D;
      a.ws_hdr[4] = gq;
      a.ws_hdr[5] = 0;
      a.ws_hdr[6] = a.pair_major;
    }
  }
  const int32_t x = static_cast<int32_t>(blockIdx.x);
  const int32_t lwg = a.pair_major ? xcd_major(x, static_cast<int32_t>(gridDim.x)) : x;
  const int32_t w = __builtin_amdgcn_readfirstlane(lwg * kWgWaves + (threadIdx.x >> 6));
  w_out = w;
  const int64_t f0 = static_cast<int64_t>(w) * C;
  f0_out = static_cast<int32_t>(min(f0, static_cast<int64_t>(total)));
  f1_out = static_cast<int32_t>(min(f0 + C, static_cast<int64_t>(total)));
  if (f0 >= total) return st;
  const int32_t f = static_cast<int32_t>(f0);
  const int32_t T = pre[a.B];  // > 0, since f0 < total = Hp T
  // pair-major: the pair row h0 of tile f and its offset r in that row; the sequence is the
  // largest b with pre[b] <= r. Sequence-major: the largest b with Hp pre[b] <= f. (pre does not
  // decrease and pre[0] = 0; the largest such b holds tiles.) Lanes test 64 evenly spaced
  // candidates at once, then the 64 (or fewer) sequences from the last one that passed.
  const int32_t h0 = a.pair_major ? f / T : 0;
  const int32_t r = a.pair_major ? f - h0 * T : f;
  const int32_t mul = a.pair_major ? 1 : a.Hp;
  const int lane = threadIdx.x & (kWave - 1);
  const int32_t S = (a.B + kWave - 1) / kWave;
  const int32_t i0 = min(lane * S, a.B - 1);
  const uint64_t m0 = __ballot(lane * S < a.B && mul * pre[i0] <= r);
  int32_t lo = (kWave - 1 - __clzll(static_cast<long long>(m0))) * S;
  if (S > 1) {
    const int32_t i1 = min(lo + lane, a.B - 1);
    const uint64_t m1 = __ballot(lane < S && lo + lane < a.B && mul * pre[i1] <= r);
    lo += kWave - 1 - __clzll(static_cast<long long>(m1));
  }
  const int32_t b0 = __builtin_amdgcn_readfirstlane(lo);
  if (a.pair_major) {
    cs_out = ChunkStart{b0, h0, h0 * T + pre[b0]};
  } else {
    const int32_t nb = pre[b0 + 1] - pre[b0];  // > 0
    const int32_t h = (f - a.Hp * pre[b0]) / nb;
    cs_out = ChunkStart{b0, h, a.Hp * pre[b0] + h * nb};
  }
  return st;
}

// Pair mode, after every wavefront of the workgroup has run its chunk of pair x and staged one
// entry per query head (none if its chunk was empty): the entries of each head are combined as
// the merge kernel combines records (maximum, rescaled sums) and the output row is stored; a
// pair with no position gets a zero row. Wavefront w takes heads w, w + 4, ...
template <int D>
__device__ __forceinline__ void combine_pair(const DecodeArgs &a, const int32_t *smem,
                                             int32_t gq) {
  const int32_t x = static_cast<int32_t>(blockIdx.x);
  const int32_t b = x / a.Hp;
  const int32_t h = x - b * a.Hp;
  const int32_t nb = smem[b + 1];  // pre[b + 1]: tiles of the pair
  const int32_t c = (nb + kWgWaves - 1) / kWgWaves;
  const int lane = threadIdx.x & (kWave - 1);
  const float *stage0 = reinterpret_cast<const float *>(smem + stage_offset(a.B));
  for (int32_t r = threadIdx.x >> 6; r < gq; r += kWgWaves) {
    float M = kFloor;
    for (int i = 0; i < kWgWaves; ++i)
      if (i * c < nb) M = fmaxf(M, stage0[(i * a.stage_rows + r) * (D + 4) + D]);
    float lsum = 0.f, o0 = 0.f, o1 = 0.f;
    for (int i = 0; i < kWgWaves; ++i) {
      if (i * c >= nb) continue;
      const float *e = stage0 + (i * a.stage_rows + r) * (D + 4);
      const float f = __builtin_amdgcn_exp2f(e[D] - M);
      lsum += e[D + 1] * f;
      o0 += e[lane] * f;
      if (D > kWave) o1 += e[lane + kWave] * f;
    }
    const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
    const int64_t row = static_cast<int64_t>(b) * a.Hq + static_cast<int64_t>(h) * gq + r;
    store_elem(a.out, row * D + lane, o0 * inv, a.out_f16);
    if (D > kWave) store_elem(a.out, row * D + lane + kWave, o1 * inv, a.out_f16);
  }
}

// Workgroup combine, after every wavefront of the workgroup has run its chunk: the cut segments
// in the edge slots are taken in chunk order (wavefront 0's start slot, its end slot, wavefront
// 1's ...); consecutive entries of one pair are combined (maximum, rescaled sums). A pair found
// whole inside the workgroup gets its output row; one that began before the workgroup's first
// tile becomes the workgroup's record in slot 0, one that goes on past its last tile the record
// in slot 1 (the merge takes workgroups as its parts). Wavefront w takes heads w, w + 4, ...
template <int D>
__device__ __forceinline__ void combine_wg(const DecodeArgs &a, int32_t *smem, int32_t gq) {
  const LdsPlan lp = lds_plan(a.B, D, a.stage_rows, gq, true, false);
  const char *lds = reinterpret_cast<const char *>(smem);
  const float *edge = reinterpret_cast<const float *>(lds + lp.edge);
  const int32_t *einfo = reinterpret_cast<const int32_t *>(lds + lp.einfo);
  const int lane = threadIdx.x & (kWave - 1);
  const int32_t x = static_cast<int32_t>(blockIdx.x);
  const int64_t wg = a.pair_major ? xcd_major(x, static_cast<int32_t>(gridDim.x)) : x;
  for (int32_t r = threadIdx.x >> 6; r < gq; r += kWgWaves) {
    bool have = false, began = false, ends = false;
    int32_t pair = -1;
    float m = kFloor, l = 0.f, o0 = 0.f, o1 = 0.f;
    auto emit = [&]() {
      if (!have) return;
      if (began || ends) {
        float *rec = a.ws_rec + ((wg * 2 + (began ? 0 : 1)) * gq + r) * (D + 4);
        rec[lane] = o0;
        if (D > kWave) rec[lane + kWave] = o1;
        if (lane == 0) {
          rec[D] = m;
          rec[D + 1] = l;
        }
      } else {
        const int32_t b = pair / a.Hp;
        const int32_t h = pair - b * a.Hp;
        const int64_t row = static_cast<int64_t>(b) * a.Hq + static_cast<int64_t>(h) * gq + r;
        const float inv = l > 0.f ? 1.0f / l : 0.f;
        store_elem(a.out, row * D + lane, o0 * inv, a.out_f16);
        if (D > kWave) store_elem(a.out, row * D + lane + kWave, o1 * inv, a.out_f16);
      }
      have = false;
    };
    for (int w = 0; w < kWgWaves; ++w) {
      for (int slot = 0; slot < 2; ++slot) {
        const int32_t flags = einfo[w * 4 + 2 * slot + 1];
        if (!(flags & 1)) continue;
        const int32_t p = einfo[w * 4 + 2 * slot];
        const float *e = edge + ((w * 2 + slot) * gq + r) * (D + 4);
        const float em = e[D], el = e[D + 1];
        const float x0 = e[lane];
        const float x1 = D > kWave ? e[lane + kWave] : 0.f;
        if (have && p == pair) {
          const float M = fmaxf(m, em);
          const float fa = __builtin_amdgcn_exp2f(m - M);
          const float fb = __builtin_amdgcn_exp2f(em - M);
          l = l * fa + el * fb;
          o0 = o0 * fa + x0 * fb;
          o1 = o1 * fa + x1 * fb;
          m = M;
        } else {
          emit();
          have = true;
          pair = p;
          m = em;
          l = el;
          o0 = x0;
          o1 = x1;
          began = w == 0 && slot == 0 && (flags & 2);
        }
        ends = w == kWgWaves - 1 && (flags & 4);
      }
    }
    emit();
  }
}

template <bool PAGED, int KV, int D, bool QF16, int GQ, bool WIN>
__global__ void __launch_bounds__(kWgThreads) decode_partial_kernel(const DecodeArgs a) {
  extern __shared__ int32_t smem[];
  using Core = VecCore<PAGED, KV, D, QF16, GQ, WIN>;
  int32_t f0, f1, w;
  ChunkStart cs;
  Stage st = partial_setup<PAGED, Core, D>(a, smem, GQ, f0, f1, cs, w);
  const Core core(threadIdx.x & (kWave - 1));
  if (a.pair_mode) {
    if (f0 < f1) run_chunk<PAGED, Core>(a, smem, smem + a.B + 1, f0, f1, cs, w, st, core, false);
    __syncthreads();
    combine_pair<D>(a, smem, GQ);
    return;
  }
  if (a.wg_combine) {
    if (f0 < f1) run_chunk<PAGED, Core>(a, smem, smem + a.B + 1, f0, f1, cs, w, st, core, true);
    __syncthreads();
    combine_wg<D>(a, smem, GQ);
    return;
  }
  if (f0 >= f1) return;
  run_chunk<PAGED, Core>(a, smem, smem + a.B + 1, f0, f1, cs, w, st, core, true);
}

template <bool PAGED, int KV, int D, bool WIN, bool APPEND>
__global__ void __launch_bounds__(kWgThreads) decode_partial_mfma_kernel(const DecodeArgs a) {
  extern __shared__ int32_t smem[];
  using Core = MfmaCore<PAGED, KV, D, WIN, APPEND>;
  int32_t f0, f1, w;
  ChunkStart cs;
  Stage st = partial_setup<PAGED, Core, D>(a, smem, a.gq, f0, f1, cs, w);
  _Float16 *vbuf = reinterpret_cast<_Float16 *>(
      reinterpret_cast<char *>(smem) +
      lds_plan(a.B, D, a.stage_rows, a.gq, a.wg_combine != 0, true).vbuf +
      (threadIdx.x >> 6) * Core::kVbufBytes);
  const Core core(threadIdx.x & (kWave - 1), vbuf);
  if (a.pair_mode) {
    if (f0 < f1) run_chunk<PAGED, Core>(a, smem, smem + a.B + 1, f0, f1, cs, w, st, core, false);
    __syncthreads();
    combine_pair<D>(a, smem, a.gq);
    return;
  }
  if (a.wg_combine) {
    if (f0 < f1) run_chunk<PAGED, Core>(a, smem, smem + a.B + 1, f0, f1, cs, w, st, core, true);
    __syncthreads();
    combine_wg<D>(a, smem, a.gq);
    return;
  }
  if (f0 >= f1) return;
  run_chunk<PAGED, Core>(a, smem, smem + a.B + 1, f0, f1, cs, w, st, core, true);
}

// ---- pass 2 ------------------------------------------------------------------------------
struct MergeArgs {
  void *out;
  const int32_t *ws_hdr;
  const int32_t *ws_pre;
  const float *ws_rec;
  int32_t B, H, G, D, out_f16;  // H: K/V heads; G: query heads per K/V head
};

constexpr int kMaxParts = 4;  // parts whose loads are in flight together (a cut pair spans 2-3)

// Every load of a wavefront's first round (the workspace header and its sequence's two prefix
// entries) is issued before any is waited for: every decision is taken from all of them at once.
// So are the record loads of each round of parts: a part index past the pair's last is clamped
// to it and its weight set to zero, so the loads need no branch. Two memory round trips for a
// pair of up to kMaxParts parts.
template <int D>
__global__ void __launch_bounds__(kWgThreads) decode_merge_kernel(const MergeArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int32_t Hq = a.H * a.G;
  // (the host keeps B * Hq below 2^31, so the row index divides in 32 bits)
  const uint32_t row = blockIdx.x * kWgWaves + (threadIdx.x >> 6);
  if (row >= static_cast<uint32_t>(a.B) * static_cast<uint32_t>(Hq)) return;
  const int64_t bh = row;
  const int32_t b = static_cast<int32_t>(row / static_cast<uint32_t>(Hq));
  const int32_t hq = static_cast<int32_t>(row % static_cast<uint32_t>(Hq));
  const int4 h03 = *reinterpret_cast<const int4 *>(a.ws_hdr);
  const int4 h47 = *reinterpret_cast<const int4 *>(a.ws_hdr + 4);
  const int32_t pb = a.ws_pre[b];
  const int32_t nb = a.ws_pre[b + 1] - pb;
  const int32_t T = a.ws_pre[a.B];  // tiles per pair row
  const int32_t C = h03.x;
  // query heads pass 1 served per wavefront (1 to 16, dividing G); the pass-1 pair of this
  // query head and its place among the pair's GQ heads
  const int32_t GQ = h47.x;
  const bool gq_ok = GQ >= 1 && GQ <= kMaxGroup && a.G % GQ == 0;
  const int32_t gq = gq_ok ? GQ : 1;
  const int32_t nsub = a.G / gq;
  const int32_t rr = hq % a.G;
  const int32_t h = (hq / a.G) * nsub + rr / gq;
  const int32_t r = rr % gq;
  // the pair's first tile in the work list (pair-major or sequence-major, as pass 1 recorded)
  const int32_t start = h47.z != 0 ? h * T + pb : a.H * nsub * pb + h * nb;
  // worker indices are clamped into the record array whatever the workspace holds
  const int32_t C1 = max(C, 1);
  const int32_t fw = min(max(start / C1, 0), kMaxWorkers - 1);
  const int32_t lw = min(max((start + nb - 1) / C1, fw), kMaxWorkers - 1);
  // h47.y != 0: pass 1 ran one workgroup per pair and wrote every row; C < 1 or a bad GQ: no
  // pass-1 record in this workspace; fw == lw: the pair was finished by pass 1
  const bool pair_mode = h47.y != 0;
  if (!pair_mode && nb == 0) {  // an empty sequence
    for (int d = lane; d < D; d += kWave) store_elem(a.out, bh * D + d, 0.f, a.out_f16);
    return;
  }
  if (pair_mode || C < 1 || nb < 0 || !gq_ok || fw == lw) return;
  constexpr int RS = D + 4;
  const int32_t nparts = lw - fw + 1;
  auto rec = [&](int32_t i) -> const float * {  // part i of the pair: the first is in slot 1
    return a.ws_rec + ((static_cast<int64_t>(fw + i) * 2 + (i == 0 ? 1 : 0)) * gq + r) * RS;
  };
  float M = kFloor, lsum = 0.f, o0 = 0.f, o1 = 0.f;
  for (int32_t i0 = 0; i0 < nparts; i0 += kMaxParts) {
    const int32_t n = min(nparts - i0, kMaxParts);
    float mi[kMaxParts], li[kMaxParts], x0[kMaxParts], x1[kMaxParts];
#pragma unroll
    for (int k = 0; k < kMaxParts; ++k) {
      const float *p = rec(i0 + min(k, n - 1));
      mi[k] = p[D];
      li[k] = p[D + 1];
      x0[k] = p[lane];
      x1[k] = D > kWave ? p[lane + kWave] : 0.f;
    }
    float Mn = M;
#pragma unroll
    for (int k = 0; k < kMaxParts; ++k) Mn = k < n ? fmaxf(Mn, mi[k]) : Mn;
    const float fo = __builtin_amdgcn_exp2f(M - Mn);
    lsum *= fo;
    o0 *= fo;
    o1 *= fo;
#pragma unroll
    for (int k = 0; k < kMaxParts; ++k) {
      if (k < n) {
        const float f = __builtin_amdgcn_exp2f(mi[k] - Mn);
        lsum += li[k] * f;
        o0 += x0[k] * f;
        o1 += x1[k] * f;
      }
    }
    M = Mn;
  }
  const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
  store_elem(a.out, bh * D + lane, o0 * inv, a.out_f16);
  if (D > kWave) store_elem(a.out, bh * D + lane + kWave, o1 * inv, a.out_f16);
}

// ---- host side ---------------------------------------------------------------------------
int device_cu_count() {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if (!cache[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

using PartialKernel = void (*)(DecodeArgs);

// How pass 1 serves G query heads per K/V head. With fp16 queries over an fp16 (or paged 8-bit)
// cache and G > 1, the matrix-core kernel serves gq heads per wavefront, the largest divisor of
// G up to 16, and each K/V byte is read G/gq times (once for G <= 16). Otherwise each query head
// is its own pair on the vector kernel and its K/V head is read once per query head.
struct GroupPlan {
  int gq;
  bool mfma;
};

inline int largest_group_divisor(int G) {
  for (int w = kMaxGroup; w > 1; --w)
    if (G % w == 0) return w;
  return 1;
}

inline GroupPlan group_plan(int G, kvc_dtype kv, bool q_f16, bool paged) {
  const bool mfma_ok = q_f16 && (kv == KVC_F16 || (paged && is_q8(kv)));
  const int w = largest_group_divisor(G);
  if (mfma_ok && w > 1) return {w, true};
  return {1, false};
}

// Records are sized for the widest group G allows, whatever the dtypes.
inline int ws_group(int G) { return largest_group_divisor(G); }

template <bool PAGED, bool QF16, int D, bool WIN>
PartialKernel pick_vec_d(kvc_dtype kv) {
  if (kv == KVC_F32) return decode_partial_kernel<PAGED, KVC_F32, D, QF16, 1, WIN>;
  if (kv == KVC_F16) return decode_partial_kernel<PAGED, KVC_F16, D, QF16, 1, WIN>;
  if constexpr (PAGED)
    if (kv == KVC_E4M3) return decode_partial_kernel<PAGED, KVC_E4M3, D, QF16, 1, WIN>;
  if constexpr (PAGED)
    if (kv == KVC_I8) return decode_partial_kernel<PAGED, KVC_I8, D, QF16, 1, WIN>;
  return nullptr;
}

// append: the instance that stores the new token's row (fp16 caches without a window); the
// other instances carry none of that code
template <bool PAGED, int D, bool WIN>
PartialKernel pick_mfma_d(kvc_dtype kv, bool append) {
  if constexpr (!WIN)
    if (append) return kv == KVC_F16 ? decode_partial_mfma_kernel<PAGED, KVC_F16, D, false, true>
                                     : nullptr;
  if (kv == KVC_F16) return decode_partial_mfma_kernel<PAGED, KVC_F16, D, WIN, false>;
  if constexpr (PAGED)
    if (kv == KVC_E4M3) return decode_partial_mfma_kernel<PAGED, KVC_E4M3, D, WIN, false>;
  if constexpr (PAGED)
    if (kv == KVC_I8) return decode_partial_mfma_kernel<PAGED, KVC_I8, D, WIN, false>;
  return nullptr;
}

template <bool PAGED, bool WIN>
PartialKernel pick_kernel_w(kvc_dtype kv, int D, bool q_f16, bool mfma, bool append) {
  if (mfma) {
    if (!q_f16) return nullptr;
    if (D == 64) return pick_mfma_d<PAGED, 64, WIN>(kv, append);
    if (D == 128) return pick_mfma_d<PAGED, 128, WIN>(kv, append);
    return nullptr;
  }
  if (D == 64)
    return q_f16 ? pick_vec_d<PAGED, true, 64, WIN>(kv) : pick_vec_d<PAGED, false, 64, WIN>(kv);
  if (D == 128)
    return q_f16 ? pick_vec_d<PAGED, true, 128, WIN>(kv) : pick_vec_d<PAGED, false, 128, WIN>(kv);
  return nullptr;
}

template <bool PAGED>
PartialKernel pick_kernel(kvc_dtype kv, int D, bool q_f16, bool mfma, bool window, bool append) {
  return window ? pick_kernel_w<PAGED, true>(kv, D, q_f16, mfma, append)
                : pick_kernel_w<PAGED, false>(kv, D, q_f16, mfma, append);
}

struct PartialPlan {
  DecodeArgs a;
  PartialKernel kern;
  int grid;
  size_t shmem;
};

// Pass-1 wavefronts per compute unit: each wavefront has about one tile of loads in flight, so
// small tiles (K+V of 16 positions) need more wavefronts to keep enough bytes in flight: 8 for
// tiles of 8 KiB or more, 12 for 4 KiB, 16 for 2 KiB (register use allows each). The matrix-core
// kernel over fp16 caches runs 4 (one workgroup, one wavefront per SIMD; with the workgroup
// combine below as well): a wavefront there serves up to 16 query heads, so each split pair costs
// up to 16 records and merges, and at the grouped-query workload (64 query heads over 8 K/V
// heads) 4 measured faster than 8 and 6.
// A contiguous cache with 8 KiB tiles (fp16, D = 128) runs 12: there a wavefront's chunk is one
// run of consecutive tiles, and at 16 sequences x 32 heads x 2048 positions 12 measured 3 %
// faster than 8 (16 slower); the paged pool at the same tile size is fastest at 8.
inline int waves_per_cu(kvc_dtype kv, int D, bool mfma, bool paged) {
  if (mfma && kv == KVC_F16) return 4;
  const int tile = 2 * kBlock * D * static_cast<int>(elt_bytes(kv));
  if (!paged && tile == 8192) return 12;
  return tile >= 8192 ? 8 : tile >= 4096 ? 12 : 16;
}

// Wavefronts of a pass-1 kernel that fit on one CU at once (from its register and LDS use),
// cached per kernel and LDS size; 0 if the runtime cannot say.
int resident_waves_per_cu(PartialKernel k, size_t shmem) {
  struct Entry {
    PartialKernel k;
    size_t shmem;
    int waves;
  };
  static std::mutex mu;
  static std::vector<Entry> cache;
  std::lock_guard<std::mutex> lock(mu);
  for (const Entry &e : cache)
    if (e.k == k && e.shmem == shmem) return e.waves;
  int blocks = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, reinterpret_cast<const void *>(k),
                                                   kWgThreads, shmem) != hipSuccess) {
    blocks = 0;
    (void)hipGetLastError();  // the failed query's error is not the caller's
  }
  if (cache.size() < 256) cache.push_back(Entry{k, shmem, blocks * kWgWaves});
  return blocks * kWgWaves;
}

// The launch shape of pass 1 from the problem's sizes alone (no pointer is read): the kernel, the
// work split, and whether one workgroup per pair finishes every row (pair mode: nothing left for
// the merge). The partial calls and kvc_decode_merge_needed take it from here, so they agree.
struct ShapePlan {
  PartialKernel kern;
  GroupPlan gp;
  int32_t Hp;           // pairs per sequence
  int stage_rows;       // staged output rows per wavefront
  size_t shmem;         // LDS bytes per workgroup
  bool pair_mode, wg_combine;
  int64_t pairs, P;     // (sequence, pair) count; wavefronts of the split
};

kvc_status plan_shape(bool paged, bool append, kvc_dtype q_dtype, kvc_dtype kv_dtype, int32_t B,
                      int32_t H, int32_t G, int32_t D, int32_t cap, int32_t max_ctx,
                      int32_t window, ShapePlan &sp) {
  if (B < 0 || H < 1 || G < 1 || max_ctx < 0 || cap < 0 || window < 0) return KVC_E_INVALID;
  if (static_cast<int64_t>(H) * G > (1 << 20)) return KVC_E_INVALID;
  if (B > kMaxBatch) return KVC_E_INVALID;
  if (!is_f32_or_f16(q_dtype)) return KVC_E_UNSUPPORTED;
  if (D != 64 && D != 128) return KVC_E_UNSUPPORTED;
  if (!paged && is_q8(kv_dtype)) return KVC_E_UNSUPPORTED;
  const bool q_f16 = q_dtype == KVC_F16;
  const GroupPlan gp = group_plan(G, kv_dtype, q_f16, paged);
  const int GQ = gp.gq;
  const int32_t Hp = H * (G / GQ);  // pairs per sequence
  const int64_t tiles_cap =
      static_cast<int64_t>(B) * Hp * ((static_cast<int64_t>(cap) + kBlock - 1) / kBlock);
  if (tiles_cap + kMaxWorkers >= INT32_MAX) return KVC_E_INVALID;
  sp = ShapePlan{};
  sp.gp = gp;
  sp.Hp = Hp;
  if (B == 0) return KVC_OK;  // nothing to launch (sp.kern stays null)

  // a window covers at most window + 15 positions' blocks
  const int64_t span = window > 0 ? std::min<int64_t>(std::min(max_ctx, cap),
                                                      static_cast<int64_t>(window) + kBlock - 1)
                                  : std::min(max_ctx, cap);
  const int64_t tiles_hint = static_cast<int64_t>(B) * Hp * ((span + kBlock - 1) / kBlock);
  PartialKernel kern =
      paged ? pick_kernel<true>(kv_dtype, D, q_f16, gp.mfma, window > 0, append)
            : pick_kernel<false>(kv_dtype, D, q_f16, gp.mfma, window > 0, append);
  if (!kern) return KVC_E_UNSUPPORTED;
  // staged rows per wavefront: a segment stages GQ rows at once; the matrix-core kernel also
  // holds one fp16 V tile per wavefront
  const int stage_rows = GQ <= kStageRows ? kStageRows : 2 * kStageRows;
  size_t shmem = lds_plan(B, D, stage_rows, GQ, false, gp.mfma).total;
  // one round of wavefronts: never more than fit on the GPU at once
  int wpc = waves_per_cu(kv_dtype, D, gp.mfma, paged);
  const int fit = resident_waves_per_cu(kern, shmem);
  if (fit > 0) wpc = std::min(wpc, fit);
  // Few, short pairs (every pair's wavefronts resident at once, at most kPairTiles tiles per
  // wavefront by the caller's bound max_ctx): one workgroup per pair, its wavefronts splitting
  // the pair's tiles and combining in LDS, so no pair is left for the merge launch.
  const int64_t pairs = static_cast<int64_t>(B) * Hp;
  const int64_t pair_span =
      window > 0 ? std::min<int64_t>(max_ctx, static_cast<int64_t>(window) + kBlock - 1) : max_ctx;
  const int64_t pair_tiles = (pair_span + kBlock - 1) / kBlock;
  const bool pair_mode = pair_tiles <= static_cast<int64_t>(kWgWaves) * kPairTiles &&
                         pairs * kWgWaves <= static_cast<int64_t>(device_cu_count()) * wpc;
  // The matrix-core kernel's wavefronts each serve up to 16 query heads, so every pair cut between
  // two wavefronts would leave up to 16 records for the merge. Its workgroups therefore combine
  // the pairs cut between their own wavefronts in LDS, and only pairs cut at workgroup edges
  // leave records. One workgroup per CU (one wavefront per SIMD): at the grouped-query workload
  // (64 query heads over 8 K/V heads, B = 32) it measured 0.9-1.3 % faster per step than two,
  // with half the workgroup edges.
  bool wg_combine = false;
  if (gp.mfma && !pair_mode) {
    const size_t sh_wg = lds_plan(B, D, stage_rows, GQ, true, true).total;
    const int fit_wg = resident_waves_per_cu(kern, sh_wg);
    if (fit_wg >= kMfmaWgWaves) {
      wg_combine = true;
      shmem = sh_wg;
      wpc = kMfmaWgWaves;
    }
  }
  int64_t P = std::min<int64_t>(kMaxWorkers, static_cast<int64_t>(device_cu_count()) * wpc);
  P = std::min<int64_t>(P, std::max<int64_t>(1, (tiles_hint + kMinChunk - 1) / kMinChunk));
  P = (P + kWgWaves - 1) / kWgWaves * kWgWaves;
  sp.kern = kern;
  sp.stage_rows = stage_rows;
  sp.shmem = shmem;
  sp.pair_mode = pair_mode;
  sp.wg_combine = wg_combine;
  sp.pairs = pairs;
  sp.P = P;
  return KVC_OK;
}

// Shared validation and planning for both layouts.
kvc_status plan_partial(bool paged, bool append, const void *q, kvc_dtype q_dtype,
                        kvc_dtype kv_dtype, const int32_t *ctx_lens, int32_t B, int32_t H,
                        int32_t G, int32_t D,
                        int32_t cap, int32_t max_ctx, int32_t window, float scale, void *out,
                        kvc_dtype out_dtype, void *workspace, size_t ws_bytes, PartialPlan &pl) {
  if (B < 0 || H < 1 || G < 1 || max_ctx < 0 || cap < 0 || window < 0) return KVC_E_INVALID;
  if (static_cast<int64_t>(H) * G > (1 << 20)) return KVC_E_INVALID;
  if (B > kMaxBatch) return KVC_E_INVALID;
  if (!is_f32_or_f16(q_dtype) || !is_f32_or_f16(out_dtype)) return KVC_E_UNSUPPORTED;
  if (D != 64 && D != 128) return KVC_E_UNSUPPORTED;
  if (!paged && is_q8(kv_dtype)) return KVC_E_UNSUPPORTED;
  if (!(scale == scale) || __builtin_isinf(scale)) return KVC_E_INVALID;
  const bool q_f16 = q_dtype == KVC_F16;
  // the sizes' own checks again in plan_shape, then (B > 0) the pointers, then the launch shape
  {
    const GroupPlan gp = group_plan(G, kv_dtype, q_f16, paged);
    const int64_t tiles_cap = static_cast<int64_t>(B) * H * (G / gp.gq) *
                              ((static_cast<int64_t>(cap) + kBlock - 1) / kBlock);
    if (tiles_cap + kMaxWorkers >= INT32_MAX) return KVC_E_INVALID;
  }
  if (B == 0) {
    pl.grid = 0;
    return KVC_OK;
  }
  if (!q || !out || !ctx_lens || !workspace) return KVC_E_INVALID;
  if (!aligned16(q) || !aligned16(out) || (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return KVC_E_INVALID;
  const WsLayout wl = ws_layout(B, D, ws_group(G));
  if (ws_bytes < wl.total) return KVC_E_INVALID;
  ShapePlan sp;
  const kvc_status ss = plan_shape(paged, append, q_dtype, kv_dtype, B, H, G, D, cap, max_ctx,
                                   window, sp);
  if (ss != KVC_OK) return ss;
  const GroupPlan gp = sp.gp;
  const int GQ = gp.gq;
  const int32_t Hp = sp.Hp;
  const PartialKernel kern = sp.kern;
  const int stage_rows = sp.stage_rows;
  const size_t shmem = sp.shmem;
  const bool pair_mode = sp.pair_mode;
  const bool wg_combine = sp.wg_combine;
  const int64_t pairs = sp.pairs;
  const int64_t P = sp.P;

  DecodeArgs &a = pl.a;
  a = DecodeArgs{};
  a.q = q;
  a.lens = ctx_lens;
  a.out = out;
  char *ws = static_cast<char *>(workspace);
  a.ws_hdr = reinterpret_cast<int32_t *>(ws);
  a.ws_pre = reinterpret_cast<int32_t *>(ws + wl.pre_off);
  a.ws_rec = reinterpret_cast<float *>(ws + wl.rec_off);
  a.B = B;
  a.H = H;
  a.G = G;
  a.nsub = G / GQ;
  a.gq = GQ;
  a.window = window;
  a.stage_rows = stage_rows;
  a.pair_mode = pair_mode ? 1 : 0;
  a.wg_combine = wg_combine ? 1 : 0;
  // Only a paged pool lets sequences share blocks, so only its list is pair-major with
  // XCD-contiguous chunks (parallel sampling: each shared block fetched about once per step
  // instead of about 4.4 times the unique bytes); a contiguous cache keeps the sequence-major
  // list, which measured 3 % faster there.
  a.pair_major = paged ? 1 : 0;
  a.Hp = Hp;
  a.Hq = H * G;
  a.cap = cap;
  a.P = static_cast<int32_t>(P);
  a.cmin = kMinChunk;
  a.q_f16 = q_f16;
  a.out_f16 = out_dtype == KVC_F16;
  a.cl2 = scale * kLog2e;
  pl.kern = kern;
  pl.grid = pair_mode ? static_cast<int>(pairs) : static_cast<int>(P / kWgWaves);
  pl.shmem = shmem;
  return KVC_OK;
}

// Device address of `scratch` on the current GPU, looked up once per device (with that device
// current) and kept; null if the runtime cannot give it.
void *scratch_address() {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void *addr[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return nullptr;
    }
    addr[dev] = p;
  }
  return addr[dev];
}

kvc_status launch_partial(const PartialPlan &pl, void *stream) {
  if (pl.grid == 0) return KVC_OK;
  hipLaunchKernelGGL(pl.kern, dim3(pl.grid), dim3(kWgThreads), pl.shmem,
                     static_cast<hipStream_t>(stream), pl.a);
  return launch_status();
}

}  // namespace kvc

using namespace kvc;

// Pass 1 for both layouts. G query heads share each K/V head (q and out have H*G heads);
// k_new/v_new non-null selects append mode (k_new/v_new hold one row per sequence and K/V
// head; not with a window); window > 0 attends only the last `window` positions of each
// sequence.
static kvc_status partial_contig(const void *q, kvc_dtype q_dtype, int32_t G, const void *k_cache,
                                 const void *v_cache, kvc_dtype kv_dtype, const int32_t *ctx_lens,
                                 const void *k_new, const void *v_new, int32_t B, int32_t H,
                                 int32_t S_max, int32_t D, int32_t max_ctx, int32_t window,
                                 float scale, void *out, kvc_dtype out_dtype, void *workspace,
                                 size_t ws_bytes, void *stream, bool *merged = nullptr) {
  if (S_max < 0) return KVC_E_INVALID;
  if (!is_f32_or_f16(kv_dtype)) return KVC_E_UNSUPPORTED;
  PartialPlan pl;
  kvc_status st = plan_partial(false, k_new != nullptr, q, q_dtype, kv_dtype, ctx_lens, B, H, G,
                               D, S_max, max_ctx,
                               window, scale, out, out_dtype, workspace, ws_bytes, pl);
  if (st != KVC_OK || pl.grid == 0) return st;
  if (!k_cache || !v_cache || !aligned16(k_cache) || !aligned16(v_cache)) return KVC_E_INVALID;
  if ((k_new != nullptr) != (v_new != nullptr)) return KVC_E_INVALID;
  if (k_new && (!aligned16(k_new) || !aligned16(v_new) || window > 0)) return KVC_E_INVALID;
  pl.a.k = static_cast<const char *>(k_cache);
  pl.a.v = static_cast<const char *>(v_cache);
  pl.a.k_new = static_cast<const char *>(k_new);
  pl.a.v_new = static_cast<const char *>(v_new);
  pl.a.seq_stride = S_max;
  if (merged) *merged = pl.a.pair_mode != 0;
  return launch_partial(pl, stream);
}

static kvc_status partial_paged(const void *q, kvc_dtype q_dtype, int32_t G,
                                const kvc_paged_layer *layer, const int32_t *block_tables,
                                int32_t max_blocks_per_seq, const int32_t *ctx_lens,
                                const void *k_new, const void *v_new, int32_t B, int32_t max_ctx,
                                int32_t window, float scale, void *out, kvc_dtype out_dtype,
                                void *workspace, size_t ws_bytes, void *stream,
                                bool *merged = nullptr) {
  if (!layer || max_blocks_per_seq < 1 || max_blocks_per_seq > INT32_MAX / kBlock)
    return KVC_E_INVALID;
  if (layer->num_blocks < 1 || layer->num_heads < 1) return KVC_E_INVALID;
  const kvc_dtype kv = layer->kv_dtype;
  if (kv != KVC_F32 && kv != KVC_F16 && !is_q8(kv)) return KVC_E_UNSUPPORTED;
  if (k_new && is_q8(kv)) return KVC_E_UNSUPPORTED;  // the block scale may change
  PartialPlan pl;
  kvc_status st = plan_partial(true, k_new != nullptr, q, q_dtype, kv, ctx_lens, B,
                               layer->num_heads, G,
                               layer->head_dim, max_blocks_per_seq * kBlock, max_ctx, window, scale,
                               out, out_dtype, workspace, ws_bytes, pl);
  if (st != KVC_OK || pl.grid == 0) return st;
  if (!block_tables || !layer->k_pool || !layer->v_pool || !aligned16(layer->k_pool) ||
      !aligned16(layer->v_pool))
    return KVC_E_INVALID;
  if (is_q8(kv) && (!layer->k_scale || !layer->v_scale)) return KVC_E_INVALID;
  if ((k_new != nullptr) != (v_new != nullptr)) return KVC_E_INVALID;
  if (k_new && (!aligned16(k_new) || !aligned16(v_new) || window > 0)) return KVC_E_INVALID;
  pl.a.k = static_cast<const char *>(layer->k_pool);
  pl.a.v = static_cast<const char *>(layer->v_pool);
  pl.a.k_scale = layer->k_scale;
  pl.a.v_scale = layer->v_scale;
  pl.a.tables = block_tables;
  pl.a.mbps = max_blocks_per_seq;
  pl.a.num_blocks = layer->num_blocks;
  pl.a.k_new = static_cast<const char *>(k_new);
  pl.a.v_new = static_cast<const char *>(v_new);
  if (merged) *merged = pl.a.pair_mode != 0;
  return launch_partial(pl, stream);
}

static kvc_status merge(int32_t B, int32_t H, int32_t G, int32_t D, void *out, kvc_dtype out_dtype,
                        void *workspace, size_t ws_bytes, void *stream) {
  if (B < 0 || H < 1 || G < 1 || B > kMaxBatch) return KVC_E_INVALID;
  if (static_cast<int64_t>(H) * G > (1 << 20)) return KVC_E_INVALID;
  if (D != 64 && D != 128) return KVC_E_UNSUPPORTED;
  if (!is_f32_or_f16(out_dtype)) return KVC_E_UNSUPPORTED;
  if (B == 0) return KVC_OK;
  if (!out || !workspace || !aligned16(out) || (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return KVC_E_INVALID;
  const WsLayout wl = ws_layout(B, D, ws_group(G));
  if (ws_bytes < wl.total) return KVC_E_INVALID;
  MergeArgs a;
  char *ws = static_cast<char *>(workspace);
  a.out = out;
  a.ws_hdr = reinterpret_cast<const int32_t *>(ws);
  a.ws_pre = reinterpret_cast<const int32_t *>(ws + wl.pre_off);
  a.ws_rec = reinterpret_cast<const float *>(ws + wl.rec_off);
  a.B = B;
  a.H = H;
  a.G = G;
  a.D = D;
  a.out_f16 = out_dtype == KVC_F16;
  const int64_t rows = static_cast<int64_t>(B) * H * G;
  if (rows > INT32_MAX) return KVC_E_INVALID;
  const int grid = static_cast<int>((rows + kWgWaves - 1) / kWgWaves);
  hipLaunchKernelGGL(D == 64 ? decode_merge_kernel<64> : decode_merge_kernel<128>, dim3(grid),
                     dim3(kWgThreads), 0, static_cast<hipStream_t>(stream), a);
  return launch_status();
}

extern "C" {

size_t kvc_decode_workspace_bytes(int32_t B, int32_t H, int32_t D) {
  if (B < 0 || H < 1 || D < 1) return 0;
  return ws_layout(B, D, 1).total;
}

size_t kvc_gqa_workspace_bytes(int32_t B, int32_t H_kv, int32_t G, int32_t D) {
  if (B < 0 || H_kv < 1 || G < 1 || D < 1) return 0;
  return ws_layout(B, D, ws_group(G)).total;
}

kvc_status kvc_decode_partial_contig(const void *q, kvc_dtype q_dtype, const void *k_cache,
                                     const void *v_cache, kvc_dtype kv_dtype,
                                     const int32_t *ctx_lens, int32_t B, int32_t H, int32_t S_max,
                                     int32_t D, int32_t max_ctx, float scale, void *out,
                                     kvc_dtype out_dtype, void *workspace, size_t ws_bytes,
                                     void *stream) {
  return partial_contig(q, q_dtype, 1, k_cache, v_cache, kv_dtype, ctx_lens, nullptr, nullptr, B,
                        H, S_max, D, max_ctx, 0, scale, out, out_dtype, workspace, ws_bytes,
                        stream);
}

kvc_status kvc_decode_partial_paged(const void *q, kvc_dtype q_dtype,
                                    const kvc_paged_layer *layer, const int32_t *block_tables,
                                    int32_t max_blocks_per_seq, const int32_t *ctx_lens, int32_t B,
                                    int32_t max_ctx, float scale, void *out, kvc_dtype out_dtype,
                                    void *workspace, size_t ws_bytes, void *stream) {
  return partial_paged(q, q_dtype, 1, layer, block_tables, max_blocks_per_seq, ctx_lens, nullptr,
                       nullptr, B, max_ctx, 0, scale, out, out_dtype, workspace, ws_bytes, stream);
}

kvc_status kvc_decode_gqa_partial_contig(const void *q, kvc_dtype q_dtype, int32_t G,
                                         const void *k_cache, const void *v_cache,
                                         kvc_dtype kv_dtype, const int32_t *ctx_lens, int32_t B,
                                         int32_t H_kv, int32_t S_max, int32_t D, int32_t max_ctx,
                                         float scale, void *out, kvc_dtype out_dtype,
                                         void *workspace, size_t ws_bytes, void *stream) {
  return partial_contig(q, q_dtype, G, k_cache, v_cache, kv_dtype, ctx_lens, nullptr, nullptr, B,
                        H_kv, S_max, D, max_ctx, 0, scale, out, out_dtype, workspace, ws_bytes,
                        stream);
}

kvc_status kvc_decode_gqa_partial_paged(const void *q, kvc_dtype q_dtype, int32_t G,
                                        const kvc_paged_layer *layer, const int32_t *block_tables,
                                        int32_t max_blocks_per_seq, const int32_t *ctx_lens,
                                        int32_t B, int32_t max_ctx, float scale, void *out,
                                        kvc_dtype out_dtype, void *workspace, size_t ws_bytes,
                                        void *stream) {
  return partial_paged(q, q_dtype, G, layer, block_tables, max_blocks_per_seq, ctx_lens, nullptr,
                       nullptr, B, max_ctx, 0, scale, out, out_dtype, workspace, ws_bytes, stream);
}

kvc_status kvc_append_decode_partial_contig(const void *q, kvc_dtype q_dtype, void *k_cache,
                                            void *v_cache, kvc_dtype kv_dtype,
                                            const int32_t *ctx_lens, const void *k_new,
                                            const void *v_new, int32_t B, int32_t H,
                                            int32_t S_max, int32_t D, int32_t max_ctx, float scale,
                                            void *out, kvc_dtype out_dtype, void *workspace,
                                            size_t ws_bytes, void *stream) {
  if (B > 0 && (!k_new || !v_new)) return KVC_E_INVALID;
  return partial_contig(q, q_dtype, 1, k_cache, v_cache, kv_dtype, ctx_lens, k_new, v_new, B, H,
                        S_max, D, max_ctx, 0, scale, out, out_dtype, workspace, ws_bytes, stream);
}

kvc_status kvc_append_decode_partial_paged(const void *q, kvc_dtype q_dtype,
                                           const kvc_paged_layer *layer,
                                           const int32_t *block_tables, int32_t max_blocks_per_seq,
                                           const int32_t *ctx_lens, const void *k_new,
                                           const void *v_new, int32_t B, int32_t max_ctx,
                                           float scale, void *out, kvc_dtype out_dtype,
                                           void *workspace, size_t ws_bytes, void *stream) {
  if (B > 0 && (!k_new || !v_new)) return KVC_E_INVALID;
  return partial_paged(q, q_dtype, 1, layer, block_tables, max_blocks_per_seq, ctx_lens, k_new,
                       v_new, B, max_ctx, 0, scale, out, out_dtype, workspace, ws_bytes, stream);
}

kvc_status kvc_decode_merge_needed(int32_t paged, int32_t append, kvc_dtype q_dtype,
                                   kvc_dtype kv_dtype, int32_t B, int32_t H, int32_t G, int32_t D,
                                   int32_t cap, int32_t max_ctx, int32_t window,
                                   int32_t *needed) {
  if (!needed) return KVC_E_INVALID;
  *needed = 0;
  if (paged) {
    if (kv_dtype != KVC_F32 && kv_dtype != KVC_F16 && !is_q8(kv_dtype)) return KVC_E_UNSUPPORTED;
    if (append && is_q8(kv_dtype)) return KVC_E_UNSUPPORTED;
  } else if (!is_f32_or_f16(kv_dtype)) {
    return KVC_E_UNSUPPORTED;
  }
  if (append && window > 0) return KVC_E_INVALID;
  ShapePlan sp;
  const kvc_status st = plan_shape(paged != 0, append != 0, q_dtype, kv_dtype, B, H, G, D, cap,
                                   max_ctx, window, sp);
  if (st != KVC_OK) return st;
  *needed = (sp.kern && !sp.pair_mode) ? 1 : 0;
  return KVC_OK;
}

kvc_status kvc_decode_merge(int32_t B, int32_t H, int32_t D, void *out, kvc_dtype out_dtype,
                            void *workspace, size_t ws_bytes, void *stream) {
  return merge(B, H, 1, D, out, out_dtype, workspace, ws_bytes, stream);
}

kvc_status kvc_decode_gqa_merge(int32_t B, int32_t H_kv, int32_t G, int32_t D, void *out,
                                kvc_dtype out_dtype, void *workspace, size_t ws_bytes,
                                void *stream) {
  return merge(B, H_kv, G, D, out, out_dtype, workspace, ws_bytes, stream);
}

kvc_status kvc_decode_attn_contig(const void *q, kvc_dtype q_dtype, const void *k_cache,
                                  const void *v_cache, kvc_dtype kv_dtype, const int32_t *ctx_lens,
                                  int32_t B, int32_t H, int32_t S_max, int32_t D, int32_t max_ctx,
                                  float scale, void *out, kvc_dtype out_dtype, void *workspace,
                                  size_t ws_bytes, void *stream) {
  bool merged = false;
  const kvc_status st =
      partial_contig(q, q_dtype, 1, k_cache, v_cache, kv_dtype, ctx_lens, nullptr, nullptr, B, H,
                     S_max, D, max_ctx, 0, scale, out, out_dtype, workspace, ws_bytes, stream,
                     &merged);
  if (st != KVC_OK || merged) return st;
  return merge(B, H, 1, D, out, out_dtype, workspace, ws_bytes, stream);
}

kvc_status kvc_decode_attn_paged(const void *q, kvc_dtype q_dtype, const kvc_paged_layer *layer,
                                 const int32_t *block_tables, int32_t max_blocks_per_seq,
                                 const int32_t *ctx_lens, int32_t B, int32_t max_ctx, float scale,
                                 void *out, kvc_dtype out_dtype, void *workspace, size_t ws_bytes,
                                 void *stream) {
  bool merged = false;
  const kvc_status st =
      partial_paged(q, q_dtype, 1, layer, block_tables, max_blocks_per_seq, ctx_lens, nullptr,
                    nullptr, B, max_ctx, 0, scale, out, out_dtype, workspace, ws_bytes, stream,
                    &merged);
  if (st != KVC_OK || merged) return st;
  return merge(B, layer->num_heads, 1, layer->head_dim, out, out_dtype, workspace, ws_bytes,
               stream);
}

kvc_status kvc_decode_attn_paged_noalloc(const void *q, kvc_dtype q_dtype,
                                         const kvc_paged_layer *layer, const int32_t *block_tables,
                                         int32_t max_blocks_per_seq, const int32_t *ctx_lens,
                                         int32_t B, int32_t max_ctx, float scale, void *out,
                                         kvc_dtype out_dtype, void *stream) {
  if (!layer || B < 0 || B > kMaxBatch) return KVC_E_INVALID;
  const int32_t D = layer->head_dim;
  if (D != 64 && D != 128) return KVC_E_UNSUPPORTED;
  if (ws_layout(B, D, 1).total > kScratchBytes) return KVC_E_INVALID;
  if (B == 0) return KVC_OK;
  void *ws = scratch_address();
  if (!ws) return KVC_E_HIP;
  return kvc_decode_attn_paged(q, q_dtype, layer, block_tables, max_blocks_per_seq, ctx_lens, B,
                               max_ctx, scale, out, out_dtype, ws, kScratchBytes, stream);
}

kvc_status kvc_decode_gqa_contig(const void *q, kvc_dtype q_dtype, int32_t G, const void *k_cache,
                                 const void *v_cache, kvc_dtype kv_dtype, const int32_t *ctx_lens,
                                 int32_t B, int32_t H_kv, int32_t S_max, int32_t D,
                                 int32_t max_ctx, float scale, void *out, kvc_dtype out_dtype,
                                 void *workspace, size_t ws_bytes, void *stream) {
  bool merged = false;
  const kvc_status st =
      partial_contig(q, q_dtype, G, k_cache, v_cache, kv_dtype, ctx_lens, nullptr, nullptr, B,
                     H_kv, S_max, D, max_ctx, 0, scale, out, out_dtype, workspace, ws_bytes,
                     stream, &merged);
  if (st != KVC_OK || merged) return st;
  return merge(B, H_kv, G, D, out, out_dtype, workspace, ws_bytes, stream);
}

kvc_status kvc_decode_gqa_paged(const void *q, kvc_dtype q_dtype, int32_t G,
                                const kvc_paged_layer *layer, const int32_t *block_tables,
                                int32_t max_blocks_per_seq, const int32_t *ctx_lens, int32_t B,
                                int32_t max_ctx, float scale, void *out, kvc_dtype out_dtype,
                                void *workspace, size_t ws_bytes, void *stream) {
  bool merged = false;
  const kvc_status st =
      partial_paged(q, q_dtype, G, layer, block_tables, max_blocks_per_seq, ctx_lens, nullptr,
                    nullptr, B, max_ctx, 0, scale, out, out_dtype, workspace, ws_bytes, stream,
                    &merged);
  if (st != KVC_OK || merged) return st;
  return merge(B, layer->num_heads, G, layer->head_dim, out, out_dtype, workspace, ws_bytes,
               stream);
}

kvc_status kvc_decode_window_partial_contig(const void *q, kvc_dtype q_dtype, int32_t G,
                                            const void *k_cache, const void *v_cache,
                                            kvc_dtype kv_dtype, const int32_t *ctx_lens,
                                            int32_t B, int32_t H_kv, int32_t S_max, int32_t D,
                                            int32_t max_ctx, int32_t window, float scale,
                                            void *out, kvc_dtype out_dtype, void *workspace,
                                            size_t ws_bytes, void *stream) {
  if (window < 1) return KVC_E_INVALID;
  return partial_contig(q, q_dtype, G, k_cache, v_cache, kv_dtype, ctx_lens, nullptr, nullptr, B,
                        H_kv, S_max, D, max_ctx, window, scale, out, out_dtype, workspace,
                        ws_bytes, stream);
}

kvc_status kvc_decode_window_partial_paged(const void *q, kvc_dtype q_dtype, int32_t G,
                                           const kvc_paged_layer *layer,
                                           const int32_t *block_tables,
                                           int32_t max_blocks_per_seq, const int32_t *ctx_lens,
                                           int32_t B, int32_t max_ctx, int32_t window,
                                           float scale, void *out, kvc_dtype out_dtype,
                                           void *workspace, size_t ws_bytes, void *stream) {
  if (window < 1) return KVC_E_INVALID;
  return partial_paged(q, q_dtype, G, layer, block_tables, max_blocks_per_seq, ctx_lens, nullptr,
                       nullptr, B, max_ctx, window, scale, out, out_dtype, workspace, ws_bytes,
                       stream);
}

kvc_status kvc_decode_window_contig(const void *q, kvc_dtype q_dtype, int32_t G,
                                    const void *k_cache, const void *v_cache, kvc_dtype kv_dtype,
                                    const int32_t *ctx_lens, int32_t B, int32_t H_kv,
                                    int32_t S_max, int32_t D, int32_t max_ctx, int32_t window,
                                    float scale, void *out, kvc_dtype out_dtype, void *workspace,
                                    size_t ws_bytes, void *stream) {
  if (window < 1) return KVC_E_INVALID;
  bool merged = false;
  const kvc_status st =
      partial_contig(q, q_dtype, G, k_cache, v_cache, kv_dtype, ctx_lens, nullptr, nullptr, B,
                     H_kv, S_max, D, max_ctx, window, scale, out, out_dtype, workspace, ws_bytes,
                     stream, &merged);
  if (st != KVC_OK || merged) return st;
  return merge(B, H_kv, G, D, out, out_dtype, workspace, ws_bytes, stream);
}

kvc_status kvc_decode_window_paged(const void *q, kvc_dtype q_dtype, int32_t G,
                                   const kvc_paged_layer *layer, const int32_t *block_tables,
                                   int32_t max_blocks_per_seq, const int32_t *ctx_lens, int32_t B,
                                   int32_t max_ctx, int32_t window, float scale, void *out,
                                   kvc_dtype out_dtype, void *workspace, size_t ws_bytes,
                                   void *stream) {
  if (window < 1) return KVC_E_INVALID;
  bool merged = false;
  const kvc_status st =
      partial_paged(q, q_dtype, G, layer, block_tables, max_blocks_per_seq, ctx_lens, nullptr,
                    nullptr, B, max_ctx, window, scale, out, out_dtype, workspace, ws_bytes,
                    stream, &merged);
  if (st != KVC_OK || merged) return st;
  return merge(B, layer->num_heads, G, layer->head_dim, out, out_dtype, workspace, ws_bytes,
               stream);
}

kvc_status kvc_append_decode_contig(const void *q, kvc_dtype q_dtype, void *k_cache,
                                    void *v_cache, kvc_dtype kv_dtype, const int32_t *ctx_lens,
                                    const void *k_new, const void *v_new, int32_t B, int32_t H,
                                    int32_t S_max, int32_t D, int32_t max_ctx, float scale,
                                    void *out, kvc_dtype out_dtype, void *workspace,
                                    size_t ws_bytes, void *stream) {
  if (B > 0 && (!k_new || !v_new)) return KVC_E_INVALID;
  bool merged = false;
  const kvc_status st =
      partial_contig(q, q_dtype, 1, k_cache, v_cache, kv_dtype, ctx_lens, k_new, v_new, B, H,
                     S_max, D, max_ctx, 0, scale, out, out_dtype, workspace, ws_bytes, stream,
                     &merged);
  if (st != KVC_OK || merged) return st;
  return merge(B, H, 1, D, out, out_dtype, workspace, ws_bytes, stream);
}

kvc_status kvc_append_decode_paged(const void *q, kvc_dtype q_dtype, const kvc_paged_layer *layer,
                                   const int32_t *block_tables, int32_t max_blocks_per_seq,
                                   const int32_t *ctx_lens, const void *k_new, const void *v_new,
                                   int32_t B, int32_t max_ctx, float scale, void *out,
                                   kvc_dtype out_dtype, void *workspace, size_t ws_bytes,
                                   void *stream) {
  if (B > 0 && (!k_new || !v_new)) return KVC_E_INVALID;
  bool merged = false;
  const kvc_status st =
      partial_paged(q, q_dtype, 1, layer, block_tables, max_blocks_per_seq, ctx_lens, k_new,
                    v_new, B, max_ctx, 0, scale, out, out_dtype, workspace, ws_bytes, stream,
                    &merged);
  if (st != KVC_OK || merged) return st;
  return merge(B, layer->num_heads, 1, layer->head_dim, out, out_dtype, workspace, ws_bytes,
               stream);
}

kvc_status kvc_append_decode_gqa_partial_contig(const void *q, kvc_dtype q_dtype, int32_t G,
                                                void *k_cache, void *v_cache, kvc_dtype kv_dtype,
                                                const int32_t *ctx_lens, const void *k_new,
                                                const void *v_new, int32_t B, int32_t H_kv,
                                                int32_t S_max, int32_t D, int32_t max_ctx,
                                                float scale, void *out, kvc_dtype out_dtype,
                                                void *workspace, size_t ws_bytes, void *stream) {
  if (B > 0 && (!k_new || !v_new)) return KVC_E_INVALID;
  return partial_contig(q, q_dtype, G, k_cache, v_cache, kv_dtype, ctx_lens, k_new, v_new, B,
                        H_kv, S_max, D, max_ctx, 0, scale, out, out_dtype, workspace, ws_bytes,
                        stream);
}

kvc_status kvc_append_decode_gqa_partial_paged(const void *q, kvc_dtype q_dtype, int32_t G,
                                               const kvc_paged_layer *layer,
                                               const int32_t *block_tables,
                                               int32_t max_blocks_per_seq, const int32_t *ctx_lens,
                                               const void *k_new, const void *v_new, int32_t B,
                                               int32_t max_ctx, float scale, void *out,
                                               kvc_dtype out_dtype, void *workspace,
                                               size_t ws_bytes, void *stream) {
  if (B > 0 && (!k_new || !v_new)) return KVC_E_INVALID;
  return partial_paged(q, q_dtype, G, layer, block_tables, max_blocks_per_seq, ctx_lens, k_new,
                       v_new, B, max_ctx, 0, scale, out, out_dtype, workspace, ws_bytes, stream);
}

kvc_status kvc_append_decode_gqa_contig(const void *q, kvc_dtype q_dtype, int32_t G,
                                        void *k_cache, void *v_cache, kvc_dtype kv_dtype,
                                        const int32_t *ctx_lens, const void *k_new,
                                        const void *v_new, int32_t B, int32_t H_kv, int32_t S_max,
                                        int32_t D, int32_t max_ctx, float scale, void *out,
                                        kvc_dtype out_dtype, void *workspace, size_t ws_bytes,
                                        void *stream) {
  if (B > 0 && (!k_new || !v_new)) return KVC_E_INVALID;
  bool merged = false;
  const kvc_status st =
      partial_contig(q, q_dtype, G, k_cache, v_cache, kv_dtype, ctx_lens, k_new, v_new, B, H_kv,
                     S_max, D, max_ctx, 0, scale, out, out_dtype, workspace, ws_bytes, stream,
                     &merged);
  if (st != KVC_OK || merged) return st;
  return merge(B, H_kv, G, D, out, out_dtype, workspace, ws_bytes, stream);
}

kvc_status kvc_append_decode_gqa_paged(const void *q, kvc_dtype q_dtype, int32_t G,
                                       const kvc_paged_layer *layer, const int32_t *block_tables,
                                       int32_t max_blocks_per_seq, const int32_t *ctx_lens,
                                       const void *k_new, const void *v_new, int32_t B,
                                       int32_t max_ctx, float scale, void *out,
                                       kvc_dtype out_dtype, void *workspace, size_t ws_bytes,
                                       void *stream) {
  if (B > 0 && (!k_new || !v_new)) return KVC_E_INVALID;
  bool merged = false;
  const kvc_status st =
      partial_paged(q, q_dtype, G, layer, block_tables, max_blocks_per_seq, ctx_lens, k_new,
                    v_new, B, max_ctx, 0, scale, out, out_dtype, workspace, ws_bytes, stream,
                    &merged);
  if (st != KVC_OK || merged) return st;
  return merge(B, layer->num_heads, G, layer->head_dim, out, out_dtype, workspace, ws_bytes,
               stream);
}

}  // extern "C"
