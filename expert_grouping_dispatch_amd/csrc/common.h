// Device-side helpers shared by the routing kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr uint32_t kSent = 0xFFFFFFFFu;
constexpr int kWave = 64;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 64-bit lane masks of the calling wave.
__device__ __forceinline__ uint64_t lanes_below() {
  return (uint64_t(1) << __lane_id()) - 1;
}

// Lanes of the wave whose `key` equals this lane's key (only among lanes with
// `valid` set): one ballot per key bit, intersected.  The caller passes
// nbits >= bit width of the largest key.
__device__ __forceinline__ uint64_t match_peers(uint32_t key, int nbits, bool valid) {
  uint64_t m = __ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (key >> b) & 1u;
    const uint64_t set = __ballot(bit);
    m &= bit ? set : ~set;
  }
  return m;
}

__device__ __forceinline__ uint64_t agent_load_u64(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void agent_store_u64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wave-wide scans with DPP lane moves (register to register, no LDS).  A
// wave64 is 4 rows of 16 lanes: row_shr:1/2/4/8 give each lane the scan over
// its row (lanes with no source read 0), then row_bcast:15 adds row r-1's last
// lane into rows 1 and 3, and row_bcast:31 adds lane 31 into rows 2 and 3.
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;

template <int kCtrl, int kRowMask>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return uint32_t(__builtin_amdgcn_update_dpp(0, int(v), kCtrl, kRowMask, 0xF, false));
}

// Inclusive wave-wide prefix sum.
__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t v) {
  v += dpp<kDppRowShr1, 0xF>(v);
  v += dpp<kDppRowShr2, 0xF>(v);
  v += dpp<kDppRowShr4, 0xF>(v);
  v += dpp<kDppRowShr8, 0xF>(v);
  v += dpp<kDppRowBcast15, 0xA>(v);
  v += dpp<kDppRowBcast31, 0xC>(v);
  return v;
}

// DPP quad_perm moves: lanes (0,1,2,3) of each group of four read lanes
// (1,0,3,2), or (2,3,0,1).
constexpr int kDppQuadSwap1 = 0xB1, kDppQuadSwap2 = 0x4E;

// Largest value over each group of four consecutive lanes, returned to all
// four.  All four lanes must be active.
__device__ __forceinline__ uint32_t quad_max(uint32_t v) {
  v = max(v, dpp<kDppQuadSwap1, 0xF>(v));
  v = max(v, dpp<kDppQuadSwap2, 0xF>(v));
  return v;
}

// Largest value over the wave, returned to every lane.
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
  v = max(v, dpp<kDppRowShr1, 0xF>(v));
  v = max(v, dpp<kDppRowShr2, 0xF>(v));
  v = max(v, dpp<kDppRowShr4, 0xF>(v));
  v = max(v, dpp<kDppRowShr8, 0xF>(v));
  v = max(v, dpp<kDppRowBcast15, 0xA>(v));
  v = max(v, dpp<kDppRowBcast31, 0xC>(v));
  return uint32_t(__builtin_amdgcn_readlane(int(v), kWave - 1));
}

}  // namespace moe
