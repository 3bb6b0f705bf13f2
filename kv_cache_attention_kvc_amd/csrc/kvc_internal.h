// Internal helpers shared by the HIP translation units of libkvc (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "kvc.h"

namespace kvc {

constexpr int kWave = 64;
constexpr int kBlock = KVC_BLOCK_SIZE;

// ---- host-side checks ------------------------------------------------------------------
inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int elt_bytes(kvc_dtype t) { return t == KVC_F32 ? 4 : (t == KVC_F16 ? 2 : 1); }

inline bool is_f32_or_f16(kvc_dtype t) { return t == KVC_F32 || t == KVC_F16; }

// 8-bit codes with one fp32 scale per block for K and one for V (e4m3 or int8).
constexpr bool is_q8(int t) { return t == KVC_E4M3 || t == KVC_I8; }

inline kvc_status launch_status() {
  return hipGetLastError() == hipSuccess ? KVC_OK : KVC_E_HIP;
}

// Compute units of the current device (cached per device ordinal).
int device_cu_count();

// ---- geometry of one (block, head) tile as read by a 64-lane wavefront -----------------
// A token row of D elements is read with 16-byte loads: LPT lanes per row, TPL rows per
// wave-wide load, LOADS loads per 16-token tile, EPL elements per lane per load.
template <int KV, int D>
struct Geo {
  static constexpr int ELT = KV == KVC_F32 ? 4 : (KV == KVC_F16 ? 2 : 1);
  static constexpr int ROW = D * ELT;
  static constexpr int LPT = ROW / 16;
  static constexpr int TPL = kWave / LPT;
  static constexpr int LOADS = kBlock / TPL;
  static constexpr int EPL = 16 / ELT;
  static constexpr int TILE = kBlock * ROW;
  static_assert(LPT >= 4 && LPT <= 32 && (LPT & (LPT - 1)) == 0, "row must span 4..32 lanes");
  static_assert(LOADS >= 1, "tile must need at least one load");
};

}  // namespace kvc
