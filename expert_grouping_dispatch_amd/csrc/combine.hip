// Stage 4: combine ("Struct_ep_combine_wait": weighted sum of the routed
// expert outputs of each token with its router weights).
//
// One workgroup per token (per part of the row when there are few rows, or
// per 128-vector part in the loop-free form); each lane owns 8 consecutive
// hidden elements (one 16-byte vector) at a time, loads that vector from up
// to kBatch expert rows at once, and accumulates in fp32 in ascending j.  Products and sums are rounded
// separately (__fmul_rn / __fadd_rn, and the library is built with
// contraction off), so the result is the same bits as the sequential
// definition.
#include "common.h"
#include "internal.h"
#include "rows.h"

namespace moe {

namespace {

constexpr int kBatch = 8;
// Vectors per lane of the whole-row kernel, and the cache policy of y loads
// and of out stores (measured on MI355X: one vector per lane, non-temporal
// loads and stores; plain loads let the next dispatch run faster but cost
// combine more).
#ifndef MOE_COMBINE_UNROLL
#define MOE_COMBINE_UNROLL 1
#endif
#ifndef MOE_COMBINE_NT_STORE
#define MOE_COMBINE_NT_STORE 1
#endif
#ifndef MOE_COMBINE_NT_LOAD
#define MOE_COMBINE_NT_LOAD 1
#endif
constexpr int kCombineMaxThreads = 1024;
// Inputs whose routed rows take less than kCombineRowsMinBytes are combined
// by the loop-free kernel in parts of kCombinePartThreads vectors; larger
// ones by whole-row workgroups (measured on MI355X: parts are faster for
// 2k-33k slot inputs, whole rows for a 7 GB stream of expert rows).
#ifndef MOE_COMBINE_PART_THREADS
#define MOE_COMBINE_PART_THREADS 128
#endif
#ifndef MOE_COMBINE_ROWS_MIN_BYTES
#define MOE_COMBINE_ROWS_MIN_BYTES (int64_t(1) << 30)
#endif
// Store policy of the loop-free kernel by working set (the routed-row
// capacity of y plus the output): from kCombinePlainMinBytes up to
// kCombinePlainMaxBytes, about what the 256 MB Infinity Cache holds, plain
// stores, which the cache absorbs while they drain (measured on MI355X: 6%
// faster on a 201 MB working set, 1.7% slower on 529 MB); outside that
// window the MOE_COMBINE_NT_STORE policy.
#ifndef MOE_COMBINE_PLAIN_MIN_BYTES
#define MOE_COMBINE_PLAIN_MIN_BYTES (int64_t(64) << 20)
#endif
#ifndef MOE_COMBINE_PLAIN_MAX_BYTES
#define MOE_COMBINE_PLAIN_MAX_BYTES (int64_t(256) << 20)
#endif
constexpr int kCombinePartThreads = MOE_COMBINE_PART_THREADS;
constexpr int64_t kCombineRowsMinBytes = MOE_COMBINE_ROWS_MIN_BYTES;
constexpr int kCombineUnroll = MOE_COMBINE_UNROLL;

// One workgroup covers a whole row: each lane owns kCombineUnroll vectors of
// 8 hidden elements, spread evenly over at most kCombineMaxThreads lanes.
int combine_threads(int h16) {
  const int per_lane = kCombineUnroll * ((h16 + kCombineUnroll * kCombineMaxThreads - 1) /
                                         (kCombineUnroll * kCombineMaxThreads));
  int t = (h16 + per_lane - 1) / per_lane;
  t = (t + 63) / 64 * 64;
  return t < 64 ? 64 : (t > kCombineMaxThreads ? kCombineMaxThreads : t);
}

__device__ __forceinline__ u32x4 load_y(const u32x4* p) {
  if constexpr (MOE_COMBINE_NT_LOAD) return __builtin_nontemporal_load(p);
  else return *p;
}

__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ void accumulate(float (&acc)[8], const u32x4& v, float wt) {
  const uint32_t word[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float lo = __uint_as_float(word[e] << 16);
    const float hi = __uint_as_float(word[e] & 0xFFFF0000u);
    acc[2 * e] = __fadd_rn(acc[2 * e], __fmul_rn(wt, lo));
    acc[2 * e + 1] = __fadd_rn(acc[2 * e + 1], __fmul_rn(wt, hi));
  }
}

// fl(scale * acc), then fl(... + residual) when a residual row is given.
__device__ __forceinline__ void epilogue(float (&acc)[8], float scale,
                                         const u32x4* __restrict__ residual, int64_t idx) {
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = __fmul_rn(scale, acc[e]);
  if (residual != nullptr) {
    const u32x4 r = residual[idx];
    const uint32_t word[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] = __fadd_rn(acc[2 * e], __uint_as_float(word[e] << 16));
      acc[2 * e + 1] = __fadd_rn(acc[2 * e + 1], __uint_as_float(word[e] & 0xFFFF0000u));
    }
  }
}

}  // namespace

// K > 0: top_k == K, positions and weights in scalar registers; K == 0: any
// top_k, compacted into LDS by wave 0 and consumed kBatch rows at a time.
// kEpilogue: out = bf16(fl(fl(scale*acc) + residual)), residual may be null
// (it never overlaps out).
template <int K, bool kEpilogue>
__global__ __launch_bounds__(kCombineMaxThreads) void k_combine(
    const u32x4* __restrict__ y, const float* __restrict__ w, const uint32_t* __restrict__ restore,
    int64_t n_rows, int h16, int top_k, float scale, const u32x4* __restrict__ residual,
    u32x4* __restrict__ out, uint32_t limit, RowSplit rs) {
  __shared__ uint32_t s_pos[K > 0 ? 1 : kMaxTopK];
  __shared__ float s_w[K > 0 ? 1 : kMaxTopK];
  __shared__ int s_n;
  constexpr int KR = K > 0 ? K : 1;
  constexpr int kRows = K > 0 ? K : kBatch;  // rows loaded at once
  const int nthreads = blockDim.x;
  const int64_t items = n_rows * rs.split;
  for (int64_t item = blockIdx.x; item < items; item += gridDim.x) {
    const int64_t t = rs.split == 1 ? item : item / rs.split;
    const int lo = int(item - t * rs.split) * rs.len;  // this workgroup's vectors [lo, hi)
    const int hi = min(h16, lo + rs.len);
    uint32_t pos[KR];
    float wt[KR];
    int n = 0;
    if constexpr (K > 0)
      uniform_slots<K, true>(restore, w, t, limit, pos, wt);
    else
      n = gather_routed(restore, w, t, top_k, limit, s_pos, s_w, &s_n);
    u32x4* dst = out + t * h16;
    for (int c0 = lo + int(threadIdx.x); c0 < hi; c0 += nthreads * kCombineUnroll) {
      float acc[kCombineUnroll][8];
#pragma unroll
      for (int u = 0; u < kCombineUnroll; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[u][e] = 0.0f;
      const int nrows = K > 0 ? K : n;
      for (int j0 = 0; j0 < nrows; j0 += kRows) {
        u32x4 v[kCombineUnroll][kRows];
#pragma unroll
        for (int jj = 0; jj < kRows; ++jj) {
          const uint32_t p = K > 0 ? pos[jj] : (j0 + jj < n ? s_pos[j0 + jj] : kSent);
          if (p != kSent) {
            const u32x4* row = y + int64_t(p) * h16;
#pragma unroll
            for (int u = 0; u < kCombineUnroll; ++u) {
              const int c = c0 + u * nthreads;
              if (c < hi) v[u][jj] = load_y(row + c);
            }
          }
        }
#pragma unroll
        for (int jj = 0; jj < kRows; ++jj) {
          const uint32_t p = K > 0 ? pos[jj] : (j0 + jj < n ? s_pos[j0 + jj] : kSent);
          if (p != kSent) {
            const float wj = K > 0 ? wt[jj] : s_w[j0 + jj];
#pragma unroll
            for (int u = 0; u < kCombineUnroll; ++u)
              if (c0 + u * nthreads < hi) accumulate(acc[u], v[u][jj], wj);
          }
        }
      }
#pragma unroll
      for (int u = 0; u < kCombineUnroll; ++u) {
        const int c = c0 + u * nthreads;
        if (c < hi) {
          if constexpr (kEpilogue) epilogue(acc[u], scale, residual, t * h16 + c);
          u32x4 o;
          o.x = bf16_rne(acc[u][0]) | (bf16_rne(acc[u][1]) << 16);
          o.y = bf16_rne(acc[u][2]) | (bf16_rne(acc[u][3]) << 16);
          o.z = bf16_rne(acc[u][4]) | (bf16_rne(acc[u][5]) << 16);
          o.w = bf16_rne(acc[u][6]) | (bf16_rne(acc[u][7]) << 16);
          if constexpr (MOE_COMBINE_NT_STORE) __builtin_nontemporal_store(o, dst + c);
          else dst[c] = o;
        }
      }
    }
    if constexpr (K == 0) __syncthreads();  // s_pos / s_w are rewritten for the next token
  }
}

// Loop-free form for top_k <= 8: one workgroup per (token, part of T
// vectors), one vector per lane; the token is item / parts from a 32-bit
// multiply-high (exact for items * parts < 2^32, which the launcher checks).
template <int K, bool kEpilogue, int T, bool kNtStore>
__global__ __launch_bounds__(T) void k_combine_parts(
    const u32x4* __restrict__ y, const float* __restrict__ w, const uint32_t* __restrict__ restore,
    int h16, float scale, const u32x4* __restrict__ residual, u32x4* __restrict__ out,
    uint32_t limit, uint32_t parts, uint32_t magic) {
  const uint32_t item = blockIdx.x;
  const uint32_t t = parts == 1 ? item : __umulhi(item, magic);
  const int c = int(item - t * parts) * T + int(threadIdx.x);
  if (c >= h16) return;
  uint32_t pos[K];
  float wt[K];
  uniform_slots<K, true>(restore, w, t, limit, pos, wt);
  u32x4 v[K];
#pragma unroll
  for (int j = 0; j < K; ++j)
    if (pos[j] != kSent) v[j] = load_y(y + uint64_t(pos[j]) * uint32_t(h16) + c);
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
#pragma unroll
  for (int j = 0; j < K; ++j)
    if (pos[j] != kSent) accumulate(acc, v[j], wt[j]);
  const uint64_t o_idx = uint64_t(t) * uint32_t(h16) + c;
  if constexpr (kEpilogue) epilogue(acc, scale, residual, int64_t(o_idx));
  u32x4 o;
  o.x = bf16_rne(acc[0]) | (bf16_rne(acc[1]) << 16);
  o.y = bf16_rne(acc[2]) | (bf16_rne(acc[3]) << 16);
  o.z = bf16_rne(acc[4]) | (bf16_rne(acc[5]) << 16);
  o.w = bf16_rne(acc[6]) | (bf16_rne(acc[7]) << 16);
  if constexpr (kNtStore) __builtin_nontemporal_store(o, out + o_idx);
  else out[o_idx] = o;
}

namespace {

template <int K>
hipError_t launch_k(const u32x4* y, const float* w, const uint32_t* restore, int64_t n_rows,
                    int h16, int top_k, bool epi, float scale, const u32x4* residual, u32x4* out,
                    uint32_t limit, hipStream_t s) {
  if constexpr (K > 0) {
    constexpr int T = kCombinePartThreads;
    const int parts = (h16 + T - 1) / T;
    const int64_t items = n_rows * parts;
    const double y_bytes = double(n_rows) * K * h16 * 16.0;
    if (y_bytes < double(kCombineRowsMinBytes) && items < (int64_t(1) << 32) / T &&
        items * parts < (int64_t(1) << 32)) {
      const uint32_t magic =
          parts == 1 ? 0u : uint32_t(((uint64_t(1) << 32) + uint64_t(parts) - 1) / uint64_t(parts));
      const double work = y_bytes + double(n_rows) * h16 * 16.0;
      const bool plain = work >= double(MOE_COMBINE_PLAIN_MIN_BYTES) && work < double(MOE_COMBINE_PLAIN_MAX_BYTES);
#define MOE_COMBINE_PARTS(EPI, NT)                                                                    \
  hipLaunchKernelGGL((k_combine_parts<K, EPI, T, NT>), dim3(uint32_t(items)), dim3(T), 0, s, y, w, \
                     restore, h16, scale, residual, out, limit, uint32_t(parts), magic)
      constexpr bool kNt = MOE_COMBINE_NT_STORE != 0;
      if (epi) {
        if (plain) MOE_COMBINE_PARTS(true, false);
        else MOE_COMBINE_PARTS(true, kNt);
      } else {
        if (plain) MOE_COMBINE_PARTS(false, false);
        else MOE_COMBINE_PARTS(false, kNt);
      }
#undef MOE_COMBINE_PARTS
      return hipGetLastError();
    }
  }
  const RowSplit rs = row_split(n_rows, h16, 128);
  const dim3 grid(row_grid(n_rows * rs.split)), block(combine_threads(rs.len));
  if (epi)
    hipLaunchKernelGGL((k_combine<K, true>), grid, block, 0, s, y, w, restore, n_rows, h16, top_k,
                       scale, residual, out, limit, rs);
  else
    hipLaunchKernelGGL((k_combine<K, false>), grid, block, 0, s, y, w, restore, n_rows, h16, top_k,
                       scale, residual, out, limit, rs);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const uint16_t* y, int64_t y_rows, const float* w,
                          const uint32_t* restore, int64_t n_rows, int hidden, int top_k,
                          bool epilogue, float scale, const uint16_t* residual, uint16_t* out,
                          hipStream_t s) {
  if (n_rows == 0) return hipSuccess;
  const u32x4* yv = reinterpret_cast<const u32x4*>(y);
  const u32x4* rv = reinterpret_cast<const u32x4*>(residual);
  u32x4* ov = reinterpret_cast<u32x4*>(out);
  const int h16 = hidden / 8;
  const uint32_t lim = position_limit(y_rows);
#define MOE_COMBINE_CASE(KK) \
  case KK: return launch_k<KK>(yv, w, restore, n_rows, h16, top_k, epilogue, scale, rv, ov, lim, s);
  switch (top_k) {
    MOE_COMBINE_CASE(1)
    MOE_COMBINE_CASE(2)
    MOE_COMBINE_CASE(3)
    MOE_COMBINE_CASE(4)
    MOE_COMBINE_CASE(5)
    MOE_COMBINE_CASE(6)
    MOE_COMBINE_CASE(7)
    MOE_COMBINE_CASE(8)
    default: return launch_k<0>(yv, w, restore, n_rows, h16, top_k, epilogue, scale, rv, ov, lim, s);
  }
#undef MOE_COMBINE_CASE
}

}  // namespace moe
