// Per-token helpers of the row kernels (dispatch and combine).
#pragma once

#include "common.h"

namespace moe {

constexpr int kMaxTopK = 1024;
// top_k up to this value is handled with per-wave uniform slot registers;
// larger top_k goes through an LDS list built by wave 0.
constexpr int kMaxUniformTopK = 8;

// Row kernels loop over tokens when there are more than kMaxRowBlocks.
constexpr int64_t kMaxRowBlocks = int64_t(1) << 20;
inline uint32_t row_grid(int64_t n_rows) {
  return uint32_t(n_rows < kMaxRowBlocks ? n_rows : kMaxRowBlocks);
}

// Combine: with few rows, one workgroup per row leaves most CUs idle and
// each workgroup moves a whole row alone.  Then each row is cut into `split` parts
// of `len` units (16-byte vectors, or MXFP4 blocks), one workgroup per part,
// aiming at about kRowSplitTarget workgroups and parts of at least
// `min_len` units.  Large inputs keep split = 1.
constexpr int64_t kRowSplitTarget = 1024;
struct RowSplit {
  int split;  // parts per row
  int len;    // units per part (the last part may be shorter)
};
inline RowSplit row_split(int64_t n_rows, int units, int min_len) {
  int split = 1;
  if (n_rows > 0 && n_rows < kRowSplitTarget) {
    const int64_t want = (kRowSplitTarget + n_rows - 1) / n_rows;
    const int64_t most = units / min_len;
    split = int(want < most ? want : most);
    if (split < 1) split = 1;
  }
  return RowSplit{split, (units + split - 1) / split};
}

// Dispatch workgroups take `lanes` consecutive units of a row (one per
// lane), so a row is cut into ceil(units / lanes) parts whatever the row count.
inline int part_count(int units, int lanes) {
  return units > lanes ? (units + lanes - 1) / lanes : 1;
}

// Positions >= limit are skipped; limit <= 0xFFFFFFFF so the sentinel is
// always skipped.
inline uint32_t position_limit(int64_t rows) {
  return rows >= int64_t(0xFFFFFFFFu) ? 0xFFFFFFFFu : uint32_t(rows);
}

// 16-byte loads and stores, non-temporal (streaming) or plain.
template <bool kNonTemporal>
__device__ __forceinline__ u32x4 load_vec(const u32x4* p) {
  if constexpr (kNonTemporal) return __builtin_nontemporal_load(p);
  else return *p;
}

template <bool kNonTemporal>
__device__ __forceinline__ void store_vec(u32x4* p, const u32x4& v) {
  if constexpr (kNonTemporal) __builtin_nontemporal_store(v, p);
  else *p = v;
}

// Host: Launch<K>::run(args...) with K = top_k for top_k <= 8 (positions in
// scalar registers), K = 0 (an LDS list) otherwise.
template <template <int> class Launch, typename... Args>
hipError_t by_top_k(int top_k, Args... args) {
  switch (top_k) {
    case 1: return Launch<1>::run(args...);
    case 2: return Launch<2>::run(args...);
    case 3: return Launch<3>::run(args...);
    case 4: return Launch<4>::run(args...);
    case 5: return Launch<5>::run(args...);
    case 6: return Launch<6>::run(args...);
    case 7: return Launch<7>::run(args...);
    case 8: return Launch<8>::run(args...);
    default: return Launch<0>::run(args...);
  }
}

// Positions restore[t*K + j] (and weights) for a compile-time K: the
// addresses are uniform across the workgroup, so every wave holds them in
// scalar registers and no LDS or barrier is needed.  Positions >= limit
// become kSent.
template <int K, bool kWeights>
__device__ __forceinline__ void uniform_slots(const uint32_t* __restrict__ restore,
                                              const float* __restrict__ w, int64_t t,
                                              uint32_t limit, uint32_t (&pos)[K], float (&wt)[K]) {
  const uint32_t* r = restore + t * K;
  uint32_t raw[K];
#pragma unroll
  for (int j = 0; j < K; ++j) raw[j] = r[j];
  if constexpr (kWeights) {
    const float* wr = w + t * K;
#pragma unroll
    for (int j = 0; j < K; ++j) wt[j] = wr[j];
  }
#pragma unroll
  for (int j = 0; j < K; ++j) pos[j] = raw[j] < limit ? raw[j] : kSent;
}

// Wave 0 collects, in ascending j, the positions restore[t*top_k + j] that
// are routed and below `limit` (and their weights, when w is given) into LDS.
// Returns the count to the whole workgroup.
__device__ __forceinline__ int gather_routed(const uint32_t* __restrict__ restore,
                                             const float* __restrict__ w, int64_t t, int top_k,
                                             uint32_t limit, uint32_t* s_pos, float* s_w,
                                             int* s_n) {
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    const uint64_t below = lanes_below();
    int n = 0;
    for (int j0 = 0; j0 < top_k; j0 += kWave) {
      const int j = j0 + lane;
      uint32_t p = kSent;
      float wt = 0.0f;
      if (j < top_k) {
        p = restore[t * top_k + j];
        if (w != nullptr) wt = w[t * top_k + j];
      }
      const bool ok = p < limit;
      const uint64_t m = __ballot(ok);
      if (ok) {
        const int r = n + __popcll(m & below);
        s_pos[r] = p;
        if (s_w != nullptr) s_w[r] = wt;
      }
      n += __popcll(m);
    }
    if (lane == 0) *s_n = n;
  }
  __syncthreads();
  return *s_n;
}

}  // namespace moe
