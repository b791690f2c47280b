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

// Inclusive wave-wide prefix sum (Hillis-Steele over shuffles).
__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t v) {
  const int lane = __lane_id();
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const uint32_t o = __shfl_up(v, d, kWave);
    if (lane >= d) v += o;
  }
  return v;
}

__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
#pragma unroll
  for (int d = kWave / 2; d > 0; d >>= 1) v = max(v, (uint32_t)__shfl_xor(v, d, kWave));
  return v;
}

}  // namespace moe
