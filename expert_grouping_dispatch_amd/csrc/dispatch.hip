// Stage 3a: dispatch token rows into the expert-contiguous buffer in bf16
// ("Struct_ep_dispatch_async_mxfp4", execute and Args: input_tokens
// [num_tokens, hidden_size] go to the experts of topk_ids).  Token-major: one
// workgroup per (token, part of the row) reads its part once and writes it to
// each of the token's routed positions, so x is read once per token instead
// of once per slot.
#include "common.h"
#include "internal.h"
#include "rows.h"

namespace moe {

namespace {

// Lanes per workgroup: each lane owns one 16-byte vector of the workgroup's
// part of the row.
#ifndef MOE_DISPATCH_THREADS
#define MOE_DISPATCH_THREADS 128
#endif
// Cache policy of the x loads (measured on MI355X: plain loads); stores by
// output size (below).
#ifndef MOE_DISPATCH_NT_LOAD
#define MOE_DISPATCH_NT_LOAD 0
#endif
// 1: streamed outputs also wait for the positions before loading x, so that
// rows with nothing routed are not read.
#ifndef MOE_DISPATCH_LAZY_STREAM
#define MOE_DISPATCH_LAZY_STREAM 0
#endif
constexpr int kDispatchThreads = MOE_DISPATCH_THREADS;
// Store policy of the bf16 kernels, by output size (measured on MI355X).
// Outputs that fit in the 256 MB Infinity Cache, [kPlainMinBytes,
// kStreamMinBytes), use plain stores, which it can absorb while they drain,
// and load x only for routed tokens.  Smaller outputs (latency-bound: plain
// stores leave dirty L2 lines to write back when the kernel ends) and larger
// ones (a stream through HBM) use non-temporal stores and load x before the
// positions arrive.
#ifndef MOE_DISPATCH_PLAIN_MIN_BYTES
#define MOE_DISPATCH_PLAIN_MIN_BYTES (int64_t(64) << 20)
#endif
#ifndef MOE_DISPATCH_STREAM_MIN_BYTES
#define MOE_DISPATCH_STREAM_MIN_BYTES (int64_t(256) << 20)
#endif
constexpr int64_t kPlainMinBytes = MOE_DISPATCH_PLAIN_MIN_BYTES;
constexpr int64_t kStreamMinBytes = MOE_DISPATCH_STREAM_MIN_BYTES;

}  // namespace

// bf16 fan-out for top_k <= 8 when the grid holds one workgroup per (token,
// part): a workgroup's whole life is one 16-byte load per lane and up to K
// stores, so it carries no loop and no 64-bit index division.  kStream:
// non-temporal stores, and x is requested before the positions so that both
// loads are in flight together (rows with nothing routed are read and
// dropped); otherwise plain stores, and x is loaded only for routed tokens.
// The token is item / parts, computed as mulhi(item, ceil(2^32 / parts)),
// which is exact for item * parts < 2^32 (the launcher checks items * parts
// < 2^32): with m = 2^32/parts + e, 0 <= e < 1, the product adds
// item*e/2^32 < 1/parts to item/parts, whose fractional part is at most
// 1 - 1/parts.
template <int K, bool kStream>
__global__ __launch_bounds__(kDispatchThreads) void k_dispatch_bf16_parts(
    const u32x4* __restrict__ x, int h16, const uint32_t* __restrict__ restore,
    u32x4* __restrict__ out, uint32_t limit, uint32_t parts, uint32_t magic) {
  const uint32_t item = blockIdx.x;
  const uint32_t t = parts == 1 ? item : __umulhi(item, magic);
  const int c = int(item - t * parts) * kDispatchThreads + int(threadIdx.x);
  if (c >= h16) return;
  const u32x4* src = x + uint64_t(t) * uint32_t(h16) + c;
  constexpr bool kEagerX = kStream && !MOE_DISPATCH_LAZY_STREAM;
  u32x4 v;
  if constexpr (kEagerX) v = load_vec<MOE_DISPATCH_NT_LOAD>(src);
  const uint32_t* r = restore + uint64_t(t) * K;
  uint32_t pos[K];
#pragma unroll
  for (int j = 0; j < K; ++j) pos[j] = r[j];
  if constexpr (!kEagerX) {
    bool any = false;
#pragma unroll
    for (int j = 0; j < K; ++j) any |= pos[j] < limit;
    if (!any) return;
    v = load_vec<MOE_DISPATCH_NT_LOAD>(src);
  }
#pragma unroll
  for (int j = 0; j < K; ++j)
    if (pos[j] < limit) store_vec<kStream>(out + uint64_t(pos[j]) * uint32_t(h16) + c, v);
}

// The general bf16 fan-out (any top_k, any row count): workgroups loop over
// (token, part) items; a part is one 16-byte vector per lane.  K > 0: top_k
// == K and the positions sit in scalar registers; K == 0: any top_k,
// positions compacted into LDS by wave 0.  kStream as in the kernel above.
template <int K, bool kStream>
__global__ __launch_bounds__(kDispatchThreads) void k_dispatch_bf16(
    const u32x4* __restrict__ x, int64_t n_rows, int h16, int top_k,
    const uint32_t* __restrict__ restore, u32x4* __restrict__ out, uint32_t limit, int parts) {
  __shared__ uint32_t s_pos[K > 0 ? 1 : kMaxTopK];
  __shared__ int s_n;
  constexpr int KR = K > 0 ? K : 1;
  const int64_t items = n_rows * parts;
  for (int64_t item = blockIdx.x; item < items; item += gridDim.x) {
    const int64_t t = parts == 1 ? item : item / parts;
    const int c = int(item - t * parts) * kDispatchThreads + int(threadIdx.x);
    const bool mine = c < h16;
    const u32x4* src = x + t * h16 + c;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (kStream && mine) v = load_vec<MOE_DISPATCH_NT_LOAD>(src);
    uint32_t pos[KR];
    float unused[KR];
    int n;
    if constexpr (K > 0) {
      uniform_slots<K, false>(restore, nullptr, t, limit, pos, unused);
      n = 0;
#pragma unroll
      for (int j = 0; j < K; ++j) n += pos[j] != kSent ? 1 : 0;
    } else {
      n = gather_routed(restore, nullptr, t, top_k, limit, s_pos, nullptr, &s_n);
    }
    if (mine && n > 0) {
      if (!kStream) v = load_vec<MOE_DISPATCH_NT_LOAD>(src);
      const int nj = K > 0 ? K : n;
#pragma unroll
      for (int j = 0; j < nj; ++j) {
        const uint32_t p = K > 0 ? pos[j] : s_pos[j];
        if (p != kSent) store_vec<kStream>(out + int64_t(p) * h16 + c, v);
      }
    }
    if constexpr (K == 0) __syncthreads();  // s_pos is rewritten for the next token
  }
}

namespace {

template <int K>
struct LaunchBf16 {
  static hipError_t run(const u32x4* x, int64_t n_rows, int h16, int top_k, const uint32_t* restore,
                        u32x4* out, uint32_t limit, hipStream_t s) {
    const int parts = part_count(h16, kDispatchThreads);
    const int64_t items = n_rows * parts;
    const double out_bytes = double(n_rows) * top_k * h16 * 16.0;
    const bool stream = out_bytes < double(kPlainMinBytes) || out_bytes >= double(kStreamMinBytes);
    if constexpr (K > 0) {
      if (items < (int64_t(1) << 32) / kDispatchThreads && items * parts < (int64_t(1) << 32)) {
        const uint32_t magic =
            parts == 1 ? 0u : uint32_t(((uint64_t(1) << 32) + uint64_t(parts) - 1) / uint64_t(parts));
        if (stream)
          hipLaunchKernelGGL((k_dispatch_bf16_parts<K, true>), dim3(uint32_t(items)),
                             dim3(kDispatchThreads), 0, s, x, h16, restore, out, limit,
                             uint32_t(parts), magic);
        else
          hipLaunchKernelGGL((k_dispatch_bf16_parts<K, false>), dim3(uint32_t(items)),
                             dim3(kDispatchThreads), 0, s, x, h16, restore, out, limit,
                             uint32_t(parts), magic);
        return hipGetLastError();
      }
    }
    if (stream)
      hipLaunchKernelGGL((k_dispatch_bf16<K, true>), dim3(row_grid(items)), dim3(kDispatchThreads),
                         0, s, x, n_rows, h16, top_k, restore, out, limit, parts);
    else
      hipLaunchKernelGGL((k_dispatch_bf16<K, false>), dim3(row_grid(items)), dim3(kDispatchThreads),
                         0, s, x, n_rows, h16, top_k, restore, out, limit, parts);
    return hipGetLastError();
  }
};

}  // namespace

hipError_t launch_dispatch_bf16(const uint16_t* x, int64_t n_rows, int hidden, int top_k,
                                const uint32_t* restore, uint16_t* out, int64_t out_rows,
                                hipStream_t s) {
  if (n_rows == 0) return hipSuccess;
  return by_top_k<LaunchBf16>(top_k, reinterpret_cast<const u32x4*>(x), n_rows, hidden / 8, top_k,
                              restore, reinterpret_cast<u32x4*>(out), position_limit(out_rows), s);
}

}  // namespace moe
