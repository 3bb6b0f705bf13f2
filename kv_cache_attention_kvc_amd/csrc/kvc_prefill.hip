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
// A workgroup of four wavefronts takes one K/V head and 128 query rows: 128 consecutive
// positions of one query head, or 64 of 2 heads, or 32 of 4 heads of a group sharing the K/V
// head; each wavefront owns 32 rows of one head. It walks the keys in steps of 64 (four cache
// blocks) from 0 to its last row's position. A step's K and V is loaded once, by all 256 threads
// with 16-byte loads (one step ahead, in registers), into LDS (two buffers, one barrier per
// step) and serves the four wavefronts. Per wavefront and step, for each 32-key tile of it:
//   S^T = K . Q^T with D/16 v_mfma_f32_32x32x16_f16: lane (h, j) = (lane/32, lane%32) feeds key
//     row perm(j) (perm swaps bits 2 and 3) and query row j and receives 16 scores of row j, keys
//     16(v/8) + 8h + v%8 of the tile; keys past the row's position are masked to -inf on the
//     steps that reach it;
//   the online softmax keeps, per row, a reference that moves only when a score passes it by the
//     headroom, and per lane the partial sum of its keys' weights;
//   O^T += V^T . P^T with D/32 x 4 v_mfma_f32_32x32x16_f16, the weights as fp16 hi + lo (about 22
//     bits): for 16 keys the hi and the lo weights each take one instruction on the same V^T
//     operand, which two transposing LDS reads deliver.
// Both tiles' score products are issued before the first tile's softmax, so that the vector
// ALUs work on one tile while the matrix cores work on the other (64-key steps measured 4-5 %
// faster than 32-key steps with two steps of loads in flight).
// LDS rows are padded (K by 16 bytes, V by 64) so that the rows one read instruction takes fall
// on distinct banks and every read offset is an immediate.
#include <algorithm>
#include <cmath>
#include <type_traits>

#include "kvc_internal.h"
#include "kvc_wave.h"

namespace kvc {

constexpr int kPfWaves = 4;
constexpr int kPfThreads = kPfWaves * kWave;
constexpr int kWaveRows = 32;                   // query rows per wavefront
constexpr int kPfRows = kWaveRows * kPfWaves;  // query rows per workgroup
constexpr int kStepBlocks = 4;                  // cache blocks per step
constexpr int kStep = kStepBlocks * kBlock;     // keys per step
constexpr int kTiles = kStep / 32;              // 32-key score tiles per step
constexpr int kMaxSeqs = 4096;
// steps whose K/V loads are in flight in registers, and the loop unroll that keeps both the LDS
// buffer (2) and the register set (kAhead) of every step a compile-time choice
constexpr int kAhead = 1;
constexpr int kUnroll = kAhead == 3 ? 6 : 2;
static_assert(kAhead >= 1 && kAhead <= 3, "prefetch depth");
static_assert(kStep % 32 == 0, "whole score tiles");
// weight headroom (log2 units): weights stay below 2^kHi, so both fp16 terms stay finite
constexpr float kHead = 7.f;
constexpr float kHi = 15.f;

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

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
  int32_t gh;  // query heads per workgroup (1, 2 or 4); positions per workgroup = 128 / gh
  int32_t gx, gy;  // workgroups per head group (an upper bound) and head groups
  int32_t out_f16;
  int32_t neg_q;  // the scale is negative: scores are taken with -q and |scale|
  float cl2;      // |scale| * log2(e) (> 0)
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

// pre[b] = workgroups before sequence b along x, pre[B] = total, in LDS. Sequence b has
// ceil(n_b / pt) tiles of pt rows and takes one workgroup per pair of them.
static __device__ void tile_prefix(const PrefillArgs &a, int32_t pt, int32_t *pre, int32_t *wsum) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid >> 6;
  const int per = (a.B + kPfThreads - 1) / kPfThreads;
  const int lo = min(a.B, tid * per);
  const int hi = min(a.B, lo + per);
  int32_t sum = 0;
  for (int i = lo; i < hi; ++i) sum += ((chunk_of(a, i).n + pt - 1) / pt + 1) / 2;
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
    run += ((chunk_of(a, i).n + pt - 1) / pt + 1) / 2;
  }
  if (tid == kPfThreads - 1) pre[a.B] = inc;
  __syncthreads();
}

// gfx950 transposing LDS read: in each group of 16 lanes, lane 4i + e receives element e of the
// 4 fp16 that lanes i, i + 4, i + 8 and i + 12 address.
static __device__ __forceinline__ f16x4 lds_read_tr(const char *p) {
  return __builtin_bit_cast(
      f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                 (__attribute__((address_space(3))) i16x4 *)(p)));
}

// The weights of 8 consecutive keys as fp16 pairs: hi[i] = (p[2i], p[2i+1]) rounded to nearest,
// lo[i] = the rounding errors p - hi rounded to nearest. v_fma_mix takes hi's half as fp16 and
// computes fma(hi, -1, p) in fp32, which is p - hi exactly, then rounds once to fp16 into the low
// or the high half. The compiler does not see these writes as vector-ALU writes, so the statement
// ends with the two wait states a matrix-core instruction reading lo needs after them.
static __device__ __forceinline__ void split8(const float (&p)[8], uint32_t (&hi)[4],
                                              uint32_t (&lo)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f16x2 h = {static_cast<_Float16>(p[2 * i]), static_cast<_Float16>(p[2 * i + 1])};
    hi[i] = __builtin_bit_cast(uint32_t, h);
  }
  asm("v_fma_mixlo_f16 %0, %4, -1.0, %8 op_sel_hi:[1,0,0]\n\t"
      "v_fma_mixlo_f16 %1, %5, -1.0, %10 op_sel_hi:[1,0,0]\n\t"
      "v_fma_mixlo_f16 %2, %6, -1.0, %12 op_sel_hi:[1,0,0]\n\t"
      "v_fma_mixlo_f16 %3, %7, -1.0, %14 op_sel_hi:[1,0,0]\n\t"
      "v_fma_mixhi_f16 %0, %4, -1.0, %9 op_sel:[1,0,0] op_sel_hi:[1,0,0]\n\t"
      "v_fma_mixhi_f16 %1, %5, -1.0, %11 op_sel:[1,0,0] op_sel_hi:[1,0,0]\n\t"
      "v_fma_mixhi_f16 %2, %6, -1.0, %13 op_sel:[1,0,0] op_sel_hi:[1,0,0]\n\t"
      "v_fma_mixhi_f16 %3, %7, -1.0, %15 op_sel:[1,0,0] op_sel_hi:[1,0,0]\n\t"
      "s_nop 1"
      : "=&v"(lo[0]), "=&v"(lo[1]), "=&v"(lo[2]), "=&v"(lo[3])
      : "v"(hi[0]), "v"(hi[1]), "v"(hi[2]), "v"(hi[3]), "v"(p[0]), "v"(p[1]), "v"(p[2]),
        "v"(p[3]), "v"(p[4]), "v"(p[5]), "v"(p[6]), "v"(p[7]));
}

template <bool PAGED, int D>
__global__ void __launch_bounds__(kPfThreads) prefill_kernel(const PrefillArgs a,
                                                             const int32_t *__restrict__ tables) {
  constexpr int ROW = D * 2;            // bytes of one fp16 row
  constexpr int NCH = D / 8;            // 16-byte columns per row
  constexpr int BLK = kBlock * ROW;     // bytes of one cache block of one head
  // LDS rows are padded so that the rows one read instruction takes fall on distinct banks:
  // K reads take 16 rows of 16 bytes, the V transposing reads 4 rows of 64 bytes.
  constexpr int KROW = ROW + 16;
  constexpr int VROW = ROW + 64;
  constexpr int VOFF = kStep * KROW;
  constexpr int BUF = kStep * (KROW + VROW);  // one step's K and V
  constexpr int NQK = D / 16;           // score MFMAs per step (16 dims each)
  constexpr int NDQ = D / 32;           // 32-dim output blocks
  constexpr int LPT = kStep * NCH / kPfThreads;  // 16-byte pieces of K (and of V) per thread
  static_assert(LPT >= 1 && kStep * NCH % kPfThreads == 0, "head dim");
  extern __shared__ int32_t smem[];
  int32_t *pre = smem;
  int32_t *wsum = smem + a.B + 1;
  char *kv_lds = reinterpret_cast<char *>(smem) + ((a.B + 1 + kPfWaves + 3) / 4) * 16;
  // kv_lds: [2 buffers][K rows (KROW bytes) | V rows (VROW bytes)], kStep rows each

  // Workgroup L runs on XCD L % 8 (round-robin dispatch). Each XCD takes a contiguous range of
  // (head group, tile) pairs, tiles fastest, so the workgroups that read one K/V head share that
  // XCD's L2.
  const uint32_t per = gridDim.x / 8;
  const uint32_t lin = (blockIdx.x % 8) * per + blockIdx.x / 8;
  if (lin >= static_cast<uint32_t>(a.gx) * static_cast<uint32_t>(a.gy)) return;
  const int32_t x = static_cast<int32_t>(lin % a.gx);
  const int32_t hgroup = static_cast<int32_t>(lin / a.gx);
  const int32_t pt = kPfRows / a.gh;
  tile_prefix(a, pt, pre, wsum);
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
  // Under the causal mask tile t (rows t pt ..) takes about t + 1 units of work: the workgroup
  // runs tile ntile - 1 - p and then tile p, so that every pair of a sequence costs about the
  // same and no long tile starts last.
  const int32_t pair = x - pre[b];
  auto run_tile = [&](const int32_t tile) {
    const int32_t rt0 = tile * pt;                  // chunk-relative rows of the workgroup
    const int32_t rt1 = min(rt0 + pt, ch.n);
    const int32_t base_pos = ch.L - ch.n;           // position of chunk row 0

    const int32_t nsub = a.G / a.gh;
    const int32_t hk = hgroup / nsub;
    const int32_t hq0 = hk * a.G + (hgroup % nsub) * a.gh;

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int w = tid >> 6;
    const int h = lane >> 5;   // half of the wavefront
    const int j = lane & 31;   // query row of the wavefront (and K row / output dim in the MFMAs)
    const int32_t hq = hq0 + w % a.gh;
    const int32_t rw0 = rt0 + kWaveRows * (w / a.gh);  // the wavefront's first row
    const int32_t nrow = max(0, min(kWaveRows, rt1 - rw0));
    const int32_t wave_first = base_pos + rw0;         // its first and last rows' positions
    const int32_t wave_last = wave_first + nrow - 1;
    const int32_t last_pos = base_pos + rt1 - 1;       // the workgroup's last position
    const int32_t nstep = last_pos / kStep + 1;

    // q operand of the score MFMAs: row j of the wavefront (rows past its end repeat its last row;
    // a wavefront with no rows reads the workgroup's first row and stores nothing), dims
    // 16c + 8h .. 16c + 8h + 7 for MFMA c; sign flipped for a negative scale
    const int32_t my_rel = nrow > 0 ? rw0 + min(j, nrow - 1) : rt0;
    uint4 qv[NQK];
    {
      const char *qr = a.q + (static_cast<int64_t>(ch.r0 + my_rel) * a.Hq + hq) * ROW;
      const uint32_t flip = a.neg_q ? 0x80008000u : 0u;
#pragma unroll
      for (int c = 0; c < NQK; ++c) {
        uint4 t = *reinterpret_cast<const uint4 *>(qr + (2 * c + h) * 16);
        t.x ^= flip;
        t.y ^= flip;
        t.z ^= flip;
        t.w ^= flip;
        qv[c] = t;
      }
    }
    const int32_t my_pos = base_pos + my_rel;

    // Step loads: piece i of thread t is 16-byte column (t + i * threads) % NCH of step row
    // (t + i * threads) / NCH, of K and of V. Rows past the sequence's end read its last row, and a
    // second block past the end reads the first block's rows (finite; those keys are masked). A
    // block whose table entry lies outside the pool is stored as zeros and its keys are masked.
    const int32_t L = ch.L;
    const int64_t kv_head_off = PAGED ? static_cast<int64_t>(hk) * BLK
                                      : (static_cast<int64_t>(b) * a.H + hk) * a.seq_stride * ROW;
    // (the table is a kernel argument of its own, marked restrict: the output stores cannot
    // alias it, so its reads stay scalar loads)
    const int32_t *trow = PAGED ? tables + static_cast<int64_t>(b) * a.mbps : nullptr;
    // kAhead steps are in flight in registers while one is computed from LDS
    uint4 kr[kAhead][LPT], vr[kAhead][LPT];
    // The table entries of the step loaded next are read one step earlier (scalar loads, kept
    // in scalar registers), and the addresses of a step are planned before the previous step's
    // LDS stores are issued, so waiting for the entries never waits for LDS work.
    struct StepPlan {
      int64_t base[kStepBlocks];  // byte offsets of the step's blocks of this head
      int32_t lim[kStepBlocks];   // last row of each block that holds a position
      int bad;                    // bit i: block i holds positions but is not in the pool
    };
    // entries of step s's blocks (kStep s <= L - 1, so its first block holds positions; a block
    // past the end takes the first block's entry)
    auto table_step = [&](int32_t s, int32_t (&p)[kStepBlocks]) {
      if constexpr (PAGED) {
        p[0] = trow[kStepBlocks * s];
#pragma unroll
        for (int i = 1; i < kStepBlocks; ++i)
          p[i] = L - s * kStep - i * kBlock > 0 ? trow[kStepBlocks * s + i] : p[0];
      } else {
#pragma unroll
        for (int i = 0; i < kStepBlocks; ++i) p[i] = 0;
      }
    };
    auto plan_step = [&](int32_t s, const int32_t (&p)[kStepBlocks]) -> StepPlan {
      StepPlan pl;
      const int32_t nv0 = min(kBlock, L - s * kStep);
      pl.bad = 0;
#pragma unroll
      for (int i = 0; i < kStepBlocks; ++i) {
        const int32_t nv = min(kBlock, L - s * kStep - i * kBlock);
        if constexpr (PAGED) {
          // a block past the end holds block 0's entry and is zeroed with it
          const bool in = static_cast<uint32_t>(p[i]) < static_cast<uint32_t>(a.num_blocks);
          pl.bad |= in ? 0 : 1 << i;
          pl.base[i] = static_cast<int64_t>(in ? p[i] : 0) * a.H * BLK + kv_head_off;
        } else {
          pl.base[i] = kv_head_off + static_cast<int64_t>(kStepBlocks * s + (nv > 0 ? i : 0)) * BLK;
        }
        pl.lim[i] = (nv > 0 ? nv : nv0) - 1;
      }
      return pl;
    };
    auto issue_step = [&](const StepPlan &pl, uint4 (&kd)[LPT], uint4 (&vd)[LPT]) {
#pragma unroll
      for (int i = 0; i < LPT; ++i) {
        const int p = tid + i * kPfThreads;
        const int row = p / NCH;
        const int sb = row >> 4;  // block of the step
        int64_t base = pl.base[0];
        int32_t lim = pl.lim[0];
#pragma unroll
        for (int k = 1; k < kStepBlocks; ++k) {
          base = sb == k ? pl.base[k] : base;
          lim = sb == k ? pl.lim[k] : lim;
        }
        const int32_t r = min(row & 15, lim);
        const int64_t off = base + r * ROW + (p % NCH) * 16;
        kd[i] = *reinterpret_cast<const uint4 *>(a.k + off);
        vd[i] = *reinterpret_cast<const uint4 *>(a.v + off);
      }
    };
    auto store_step = [&](char *buf, int bad, uint4 (&kd)[LPT], uint4 (&vd)[LPT]) {
      if (bad != 0) {
#pragma unroll
        for (int i = 0; i < LPT; ++i) {
          const int sb = ((tid + i * kPfThreads) / NCH) >> 4;
          if ((bad >> sb) & 1) kd[i] = vd[i] = make_uint4(0, 0, 0, 0);
        }
      }
#pragma unroll
      for (int i = 0; i < LPT; ++i) {
        const int p = tid + i * kPfThreads;
        const int row = p / NCH, col = p % NCH;
        *reinterpret_cast<uint4 *>(buf + row * KROW + col * 16) = kd[i];
        *reinterpret_cast<uint4 *>(buf + VOFF + row * VROW + col * 16) = vd[i];
      }
    };

    // Score MFMA: the A operand row j is key perm(j), perm swapping bits 2 and 3, so that lane
    // (h, j)'s 16 scores (element v: A row 8(v/4) + 4h + v%4) are keys 16(v/8) + 8h + v%8 of query
    // row j: two runs of 8 consecutive keys, one per cache block.
    const int kperm = (j & ~12) | ((j & 4) << 1) | ((j & 8) >> 1);
    const int k_lds = kperm * KROW + h * 16;
    // V^T operand of the output MFMAs: lane (h, j) needs V[16a + 8h + t][32dq + j], t = 0..7,
    // fetched as two transposing reads of 4 keys; lane s of its 16-lane group addresses key row
    // 16a + 8h + 4r + s/4, dims 32dq + 16(j/16) + 4(s%4) .. + 3 for read r.
    const int s16 = lane & 15;
    const int v_lds = VOFF + (8 * h + (s16 >> 2)) * VROW + (16 * (j >> 4) + 4 * (s16 & 3)) * 2;

    f32x16 o[NDQ];
#pragma unroll
    for (int dq = 0; dq < NDQ; ++dq)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[dq][e] = 0.f;
    float m = kFloor, l = 0.f;
    float mt = kFloor + kHi;  // m + kHi
    const float cl2 = a.cl2;

    // The wavefront's share of one step (keys kStep * s ..), its K and V in LDS at `buf`. MASK:
    // the step holds keys past some row's position or blocks outside the pool (bits of `bad`).
    // The scores of every 32-key tile are issued first; the softmax of tile t then runs on the
    // vector ALUs while the matrix cores still work on the scores of tile t + 1 or on the
    // products of tile t - 1.
    auto compute = [&](const char *buf, int32_t s, auto mask_tag, int bad) {
      constexpr bool MASK = decltype(mask_tag)::value;
      // tiles holding a key at or before the wavefront's last row (every tile unless MASK)
      const int nt = MASK ? min(kTiles, (wave_last - s * kStep) / 32 + 1) : kTiles;
      // (a skipped tile's scores are never read; the first product of a tile takes a zero
      // accumulator as an immediate)
      f32x16 sc[kTiles];
#pragma unroll
      for (int t = 0; t < kTiles; ++t) {
        if (MASK && t >= nt) continue;
#pragma unroll
        for (int c = 0; c < NQK; ++c) {
          const uint4 kv = *reinterpret_cast<const uint4 *>(buf + t * 32 * KROW + k_lds + c * 32);
          sc[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_f16x8(kv), as_f16x8(qv[c]),
                                                         c == 0 ? f32x16{} : sc[t], 0, 0, 0);
        }
      }
#pragma unroll
      for (int t = 0; t < kTiles; ++t) {
        if (MASK && t >= nt) break;
        if constexpr (MASK) {
          // key 32t + 16(v/8) + 8h + v%8 of the step (block 2t + v/8) is kept when at or before
          // the row's position
          const int32_t lim = my_pos - s * kStep - 32 * t - 8 * h;
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const bool keep =
                16 * (v >> 3) + (v & 7) <= lim && !((bad >> (2 * t + (v >> 3))) & 1);
            sc[t][v] = keep ? sc[t][v] : -__builtin_inff();
          }
        }
        float mx = sc[t][0];
#pragma unroll
        for (int v = 1; v < 16; ++v) mx = fmaxf(mx, sc[t][v]);
        // a score that would put a weight above 2^kHi moves the row's reference (rare)
        if (__ballot(mx * cl2 > mt) != 0) {
          float u, w2;
          lane_pair<32>(mx * cl2, u, w2);
          const float rmax = fmaxf(u, w2);
          const float mnew = rmax > mt ? rmax - kHead : m;
          const float f = __builtin_amdgcn_exp2f(m - mnew);
          l *= f;
#pragma unroll
          for (int dq = 0; dq < NDQ; ++dq) o[dq] *= f;
          m = mnew;
          mt = m + kHi;
        }
        const float nm = -m;
        uint32_t ph[2][4], pl[2][4];  // keys 16 a16 + 8h + 2i, + 1 as fp16 pairs, hi and lo terms
#pragma unroll
        for (int a16 = 0; a16 < 2; ++a16) {
          float p[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[t][8 * a16 + i], cl2, nm));
            l += p[i];
          }
          split8(p, ph[a16], pl[a16]);
        }
        // O^T += V^T P^T: per 32 dims and 16 keys, the hi and the lo weights share one V^T
        // operand
#pragma unroll
        for (int a16 = 0; a16 < 2; ++a16) {
#pragma unroll
          for (int dq = 0; dq < NDQ; ++dq) {
            const char *vp = buf + v_lds + (2 * t + a16) * 16 * VROW + dq * 64;
            const f16x4 v0 = lds_read_tr(vp);
            const f16x4 v1 = lds_read_tr(vp + 4 * VROW);
            const f16x8 va = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
            const f16x8 bh = __builtin_bit_cast(
                f16x8, make_uint4(ph[a16][0], ph[a16][1], ph[a16][2], ph[a16][3]));
            const f16x8 bl = __builtin_bit_cast(
                f16x8, make_uint4(pl[a16][0], pl[a16][1], pl[a16][2], pl[a16][3]));
            o[dq] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va, bh, o[dq], 0, 0, 0);
            o[dq] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va, bl, o[dq], 0, 0, 0);
          }
        }
      }
    };

    // One step s, its K/V in LDS buffer s % 2 and in flight in register set s % kAhead: store that
    // set, reload it with step s + kAhead, one barrier, compute. The LDS buffer written here was
    // last read two steps ago, before every wavefront passed the previous barrier.
    int bad_q[kAhead];
    int32_t tp[kStepBlocks];  // table entries of the step loaded next
#pragma unroll
    for (int r = 0; r < kAhead; ++r) {
      bad_q[r] = 0;
      if (r < nstep) {
        table_step(r, tp);
        const StepPlan pl = plan_step(r, tp);
        issue_step(pl, kr[r], vr[r]);
        bad_q[r] = pl.bad;
      }
    }
    if (kAhead < nstep) table_step(kAhead, tp);
    auto step = [&](auto u_tag, int32_t s) {
      constexpr int U = decltype(u_tag)::value;
      constexpr int RS = U % kAhead;
      char *buf = kv_lds + (U % 2) * BUF;
      const int bad = bad_q[RS];
      const bool more = s + kAhead < nstep;
      StepPlan pl{};
      if (more) pl = plan_step(s + kAhead, tp);
      store_step(buf, bad, kr[RS], vr[RS]);
      if (more) {
        issue_step(pl, kr[RS], vr[RS]);
        bad_q[RS] = pl.bad;
        if (s + kAhead + 1 < nstep) table_step(s + kAhead + 1, tp);
      }
      __syncthreads();
      if (nrow > 0 && s * kStep <= wave_last) {
        if (bad != 0 || s * kStep + kStep - 1 > wave_first)
          compute(buf, s, std::true_type{}, bad);
        else
          compute(buf, s, std::false_type{}, 0);
      }
    };
    // unrolled over a whole number of LDS buffer and register set cycles
    auto steps = [&](int32_t s0, auto... us) {
      ((s0 + decltype(us)::value < nstep ? step(us, s0 + decltype(us)::value) : void()), ...);
    };
    for (int32_t s0 = 0; s0 < nstep; s0 += kUnroll) {
      if constexpr (kUnroll == 2)
        steps(s0, std::integral_constant<int, 0>{}, std::integral_constant<int, 1>{});
      else
        steps(s0, std::integral_constant<int, 0>{}, std::integral_constant<int, 1>{},
              std::integral_constant<int, 2>{}, std::integral_constant<int, 3>{},
              std::integral_constant<int, 4>{}, std::integral_constant<int, 5>{});
    }
    if (nrow == 0) return;
    {
      float u, t;
      lane_pair<32>(l, u, t);
      l = u + t;
    }
    if (j >= nrow) return;
    const float inv = l > 0.f ? 1.0f / l : 0.f;
    // lane (h, j) holds dims 32dq + 8(v/4) + 4h + v%4 of row j
    const int64_t orow = (static_cast<int64_t>(ch.r0 + rw0 + j) * a.Hq + hq) * D;
#pragma unroll
    for (int dq = 0; dq < NDQ; ++dq) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int64_t i = orow + 32 * dq + 8 * q4 + 4 * h;
        const f32x4 r = {o[dq][4 * q4] * inv, o[dq][4 * q4 + 1] * inv, o[dq][4 * q4 + 2] * inv,
                         o[dq][4 * q4 + 3] * inv};
        if (a.out_f16) {
          const f16x4 hv = {static_cast<_Float16>(r[0]), static_cast<_Float16>(r[1]),
                            static_cast<_Float16>(r[2]), static_cast<_Float16>(r[3])};
          *reinterpret_cast<f16x4 *>(static_cast<_Float16 *>(a.out) + i) = hv;
        } else {
          *reinterpret_cast<f32x4 *>(static_cast<float *>(a.out) + i) = r;
        }
      }
    }
  };
  run_tile(ntile - 1 - pair);
  if (pair < ntile - 1 - pair) {
    __syncthreads();  // the LDS buffers of the first tile are free again
    run_tile(pair);
  }
}

using PrefillKernel = void (*)(PrefillArgs, const int32_t *);

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
  // scores are taken as (sign(scale) q) . k times |scale| log2(e); a zero scale takes the
  // smallest normal float, which leaves every weight of a row equal, as a zero scale does
  a.neg_q = scale < 0.f;
  a.cl2 = scale == 0.f ? 1.17549435e-38f : fabsf(scale) * kLog2e;
  const int32_t pt = kPfRows / a.gh;
  // an upper bound on the workgroups along x: sum_b ceil(ceil(n_b / pt) / 2) <= total / 2pt + B
  const int64_t gx = (static_cast<int64_t>(a.total) + 2 * pt - 1) / (2 * pt) + a.B;
  const int64_t gy = static_cast<int64_t>(a.H) * (a.G / a.gh);
  const int64_t n8 = (gx * gy + 7) / 8 * 8;  // a multiple of the 8 XCDs
  if (n8 > INT32_MAX) return KVC_E_INVALID;
  a.gx = static_cast<int32_t>(gx);
  a.gy = static_cast<int32_t>(gy);
  const size_t shmem = static_cast<size_t>((a.B + 1 + kPfWaves + 3) / 4) * 16 +
                       static_cast<size_t>(2) * kStep * (2 * (2 * D) + 16 + 64);
  PrefillKernel kern = paged ? pick_prefill<true>(D) : pick_prefill<false>(D);
  if (!kern) return KVC_E_UNSUPPORTED;
  hipLaunchKernelGGL(kern, dim3(static_cast<uint32_t>(n8)), dim3(kPfThreads), shmem,
                     static_cast<hipStream_t>(stream), a, a.tables);
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
