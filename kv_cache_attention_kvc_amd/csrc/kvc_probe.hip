// Read-stream probe: what the memory system delivers for a given list of pieces when nothing
// else is done with them. Decode attention is bound by the bandwidth of reading the cache
// ("LLM Inference Acceleration -- KV Cache", section 6.3), so its rate is compared with a pure
// read of exactly the pieces it reads (the (block, head) tiles of K and V in work-list order),
// and with a sequential read of the same number of bytes.
//
// Each wavefront reads a contiguous run of the list, one piece after another, with the next
// piece's loads in flight while the current one is folded into a checksum (so no load is dead).
// Loads are 16-byte non-temporal loads, one wave-wide load per KiB, as in pass 1.
#include "kvc_internal.h"
#include "kvc_wave.h"

namespace kvc {
namespace {

constexpr int kProbeWaves = 4;
constexpr int kProbeThreads = kWave * kProbeWaves;
constexpr int kProbeMaxWaves = 1 << 16;

template <int KB, bool TWO>
struct Piece {
  uint4 r[TWO ? 2 * KB : KB];
};

// The piece at offset o of a (and of b), or, when not live, a stand-in: the first 256 bytes of
// a, which every wavefront shares (cached after the first read), so it adds no traffic.
template <int KB, bool TWO>
__device__ __forceinline__ void fetch_piece(const char *a, const char *b, int64_t o, bool live,
                                            int lane, Piece<KB, TWO> &p) {
  const int64_t base = live ? o : 0;
  const int lo = live ? lane * 16 : (lane & 15) * 16;
#pragma unroll
  for (int k = 0; k < KB; ++k) {
    const int64_t ko = base + (live ? k * 1024 : 0) + lo;
    p.r[k] = load_stream(a + ko);
    if constexpr (TWO) p.r[KB + k] = load_stream(b + ko);
  }
}

template <int KB, bool TWO>
__device__ __forceinline__ void fold_piece(const Piece<KB, TWO> &p, uint32_t &acc) {
#pragma unroll
  for (int k = 0; k < (TWO ? 2 * KB : KB); ++k) acc ^= p.r[k].x ^ p.r[k].y ^ p.r[k].z ^ p.r[k].w;
}

template <int KB, bool TWO>
__global__ void __launch_bounds__(kProbeThreads)
    read_pieces_kernel(const char *a, const char *b, const int64_t *off, int32_t n, int32_t C,
                       uint32_t *sink) {
  const int lane = threadIdx.x & (kWave - 1);
  const int32_t w = blockIdx.x * kProbeWaves + (threadIdx.x >> 6);
  const int64_t i0 = static_cast<int64_t>(w) * C;
  const int64_t i1 = i0 + C < n ? i0 + C : n;
  uint32_t acc = 0;
  if (i0 < i1) {
    Piece<KB, TWO> pa, pb;
    int64_t i = i0;
    fetch_piece<KB, TWO>(a, b, off[i0], true, lane, pa);
    // every step issues one fetch of the same shape (after the run's last piece, the stand-in)
    auto step = [&](Piece<KB, TWO> &cur, Piece<KB, TWO> &nxt) -> bool {
      const bool more = i + 1 < i1;
      fetch_piece<KB, TWO>(a, b, off[more ? i + 1 : i], more, lane, nxt);
      fold_piece<KB, TWO>(cur, acc);
      ++i;
      return more;
    };
    for (;;) {
      if (!step(pa, pb)) {
        fold_piece<KB, TWO>(pb, acc);
        break;
      }
      if (!step(pb, pa)) {
        fold_piece<KB, TWO>(pa, acc);
        break;
      }
    }
  }
  // every lane's checksum reaches the stored word, so every lane's loads are live
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) acc ^= __shfl_xor(acc, o);
  if (lane == 0) sink[w] = acc;
}

using ProbeKernel = void (*)(const char *, const char *, const int64_t *, int32_t, int32_t,
                             uint32_t *);

template <bool TWO>
ProbeKernel pick_probe(int kb) {
  switch (kb) {
    case 1: return read_pieces_kernel<1, TWO>;
    case 2: return read_pieces_kernel<2, TWO>;
    case 4: return read_pieces_kernel<4, TWO>;
    case 8: return read_pieces_kernel<8, TWO>;
    default: return nullptr;
  }
}

}  // namespace
}  // namespace kvc

using namespace kvc;

extern "C" kvc_status kvc_read_pieces(const void *a, const void *b, const int64_t *offsets,
                                      int32_t n, int32_t piece_bytes, int32_t waves_per_cu,
                                      uint32_t *sink, size_t sink_words, void *stream) {
  if (n < 0 || waves_per_cu < 1 || waves_per_cu > 32) return KVC_E_INVALID;
  if (piece_bytes != 1024 && piece_bytes != 2048 && piece_bytes != 4096 && piece_bytes != 8192)
    return KVC_E_UNSUPPORTED;
  if (n == 0) return KVC_OK;
  if (!a || !offsets || !sink || !aligned16(a) || (b && !aligned16(b))) return KVC_E_INVALID;
  int64_t P = static_cast<int64_t>(device_cu_count()) * waves_per_cu;
  P = (P + kProbeWaves - 1) / kProbeWaves * kProbeWaves;
  if (P > kProbeMaxWaves || sink_words < static_cast<size_t>(P)) return KVC_E_INVALID;
  const int64_t C = (static_cast<int64_t>(n) + P - 1) / P;
  const ProbeKernel k = b ? pick_probe<true>(piece_bytes / 1024) : pick_probe<false>(piece_bytes / 1024);
  hipLaunchKernelGGL(k, dim3(static_cast<unsigned>(P / kProbeWaves)), dim3(kProbeThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const char *>(a),
                     static_cast<const char *>(b), offsets, n, static_cast<int32_t>(C), sink);
  return launch_status();
}
