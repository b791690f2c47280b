// Stage 4: combine ("Struct_ep_combine_wait": weighted sum of the routed
// expert outputs of each token with its router weights).
//
// One workgroup per token; each lane owns 8 consecutive hidden elements (one
// 16-byte vector) at a time, loads that vector from up to kBatch expert rows
// at once, and accumulates in fp32 in ascending j.  Products and sums are
// rounded separately (__fmul_rn / __fadd_rn, and the library is built with
// contraction off), so the result is the same bits as the sequential
// definition.
#include "common.h"
#include "internal.h"
#include "rows.h"

namespace moe {

namespace {

constexpr int kBatch = 8;

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

}  // namespace

__global__ __launch_bounds__(kRowThreads) void k_combine(
    const u32x4* __restrict__ y, const float* __restrict__ w, const uint32_t* __restrict__ restore,
    int64_t n_rows, int h16, int top_k, u32x4* __restrict__ out, uint32_t limit) {
  __shared__ uint32_t s_pos[kMaxTopK];
  __shared__ float s_w[kMaxTopK];
  __shared__ int s_n;
  for (int64_t t = blockIdx.x; t < n_rows; t += gridDim.x) {
  const int n = gather_routed(restore, w, t, top_k, limit, s_pos, s_w, &s_n);
  u32x4* dst = out + t * h16;
  for (int c = threadIdx.x; c < h16; c += kRowThreads) {
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
    for (int j0 = 0; j0 < n; j0 += kBatch) {
      u32x4 v[kBatch];
#pragma unroll
      for (int jj = 0; jj < kBatch; ++jj)
        if (j0 + jj < n) v[jj] = __builtin_nontemporal_load(y + int64_t(s_pos[j0 + jj]) * h16 + c);
#pragma unroll
      for (int jj = 0; jj < kBatch; ++jj)
        if (j0 + jj < n) accumulate(acc, v[jj], s_w[j0 + jj]);
    }
    u32x4 o;
    o.x = bf16_rne(acc[0]) | (bf16_rne(acc[1]) << 16);
    o.y = bf16_rne(acc[2]) | (bf16_rne(acc[3]) << 16);
    o.z = bf16_rne(acc[4]) | (bf16_rne(acc[5]) << 16);
    o.w = bf16_rne(acc[6]) | (bf16_rne(acc[7]) << 16);
    __builtin_nontemporal_store(o, dst + c);
  }
  __syncthreads();  // s_pos / s_w are rewritten for the next token
  }
}

hipError_t launch_combine(const uint16_t* y, int64_t y_rows, const float* w,
                          const uint32_t* restore, int64_t n_rows, int hidden, int top_k,
                          uint16_t* out, hipStream_t s) {
  if (n_rows == 0) return hipSuccess;
  hipLaunchKernelGGL(k_combine, dim3(row_grid(n_rows)), dim3(kRowThreads), 0, s,
                     reinterpret_cast<const u32x4*>(y), w, restore, n_rows, hidden / 8, top_k,
                     reinterpret_cast<u32x4*>(out), position_limit(y_rows));
  return hipGetLastError();
}

}  // namespace moe
