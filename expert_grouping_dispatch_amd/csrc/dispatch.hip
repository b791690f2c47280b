// Stage 3: dispatch token rows into the expert-contiguous buffer, as bf16 or
// as MXFP4 ("Struct_ep_dispatch_async_mxfp4": input_tokens [num_tokens,
// hidden_size] go to the experts of topk_ids; FP4 quants travel with their
// scales).  Token-major: one workgroup per (token, part of the row) reads its
// part once and writes it to each of the token's routed positions, so x is
// read once per token instead of once per slot.
#include "common.h"
#include "internal.h"
#include "rows.h"

namespace moe {

namespace {

// Lanes per workgroup.  bf16: each lane owns one 16-byte vector of the
// workgroup's part of the row; MXFP4: one 32-element block at a time.
#ifndef MOE_DISPATCH_THREADS
#define MOE_DISPATCH_THREADS 128
#endif
#ifndef MOE_MXFP4_THREADS
#define MOE_MXFP4_THREADS 256
#endif
// Cache policy (measured on MI355X): plain loads of x; bf16 stores by output
// size (below); non-temporal stores for the separate MXFP4 payload rows,
// which are 128-byte aligned.
#ifndef MOE_DISPATCH_NT_LOAD
#define MOE_DISPATCH_NT_LOAD 0
#endif
#ifndef MOE_MXFP4_NT_LOAD
#define MOE_MXFP4_NT_LOAD 0
#endif
#ifndef MOE_MXFP4_NT_STORE
#define MOE_MXFP4_NT_STORE 1
#endif
// Packed rows (17 bytes per block) are not 128-byte aligned, so adjacent
// rows share cache lines; plain stores let the caches merge those lines.
#ifndef MOE_MXFP4_PACKED_NT_STORE
#define MOE_MXFP4_PACKED_NT_STORE 0
#endif
// Outputs (payload and scales) of [MIN, MAX) bytes, with top_k <= 8, load
// each lane's first block of x before the token's positions arrive, so that
// the two loads are in flight together (rows with nothing routed are then
// read and dropped).  Measured on MI355X: 3.7% faster on a 125 MB output; no
// faster on 3-30 MB outputs, which would only read more; 2.5% slower on a
// 1.9 GB one, where the wasted reads and the registers this takes cost more
// than the overlap saves.
#ifndef MOE_MXFP4_EAGER_MIN_BYTES
#define MOE_MXFP4_EAGER_MIN_BYTES (int64_t(64) << 20)
#endif
#ifndef MOE_MXFP4_EAGER_MAX_BYTES
#define MOE_MXFP4_EAGER_MAX_BYTES (int64_t(256) << 20)
#endif
constexpr int kDispatchThreads = MOE_DISPATCH_THREADS;
constexpr int kMxThreads = MOE_MXFP4_THREADS;
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

// E8M0 exponent of a 32-element block from the largest magnitude, given as
// the 15-bit magnitude of a bf16 pattern: floor(log2 amax) - 2, clamped to
// [-127, 127]; -127 for an all-zero block.  kEven rounds amax to one
// mantissa bit (ties away) first: the floor gains 1 when the 7-bit mantissa
// is >= 0.75 (0x60).  Subnormal amax clamps to -127 either way.
template <bool kEven>
__device__ __forceinline__ int mx_scale_exponent(uint32_t amax) {
  if (amax == 0) return -127;
  const int ef = int(amax >> 7);
  int fl = ef > 0 ? ef - 127 : -133 + (31 - __clz(amax));  // subnormal: m * 2^-133
  if (kEven && ef > 0 && (amax & 0x7Fu) >= 0x60u) fl += 1;
  const int se = fl - 2;
  return se < -127 ? -127 : se;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Four packed E2M1 bytes from four bf16 pairs with the gfx950 scaled
// conversion (v_cvt_scalef32_pk_fp4_bf16): each byte holds code(x / scale)
// of its pair, the first element in the low nibble.  Its rounding (nearest,
// ties to the even code, saturation at 6, sign kept on zero) equals the
// E2M1 rule of this dispatch for every finite bf16 value |x| < 8 * scale,
// which covers every element of a block whose scale comes from the block
// maximum.
__device__ __forceinline__ uint32_t e2m1_word(const uint32_t* w, float scale) {
  uint32_t r = 0u;
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2, w[0]), scale, 0);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2, w[1]), scale, 1);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2, w[2]), scale, 2);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2, w[3]), scale, 3);
  return r;
}

// 2^se as an fp32 value for se in [-127, 127] (2^-127 is the subnormal 0x00400000).
__device__ __forceinline__ float pow2_f32(int se) {
  return __uint_as_float(se >= -126 ? uint32_t(se + 127) << 23 : 0x00400000u);
}

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
  u32x4 v;
  if constexpr (kStream) v = load_vec<MOE_DISPATCH_NT_LOAD>(src);
  const uint32_t* r = restore + uint64_t(t) * K;
  uint32_t pos[K];
#pragma unroll
  for (int j = 0; j < K; ++j) pos[j] = r[j];
  if constexpr (!kStream) {
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

// One lane per 32-element block: 4 x 16-byte loads, 16 bytes of payload and
// one scale byte per routed position.  kPacked: one row of 17*nblk bytes per
// slot, the 16*nblk payload bytes first and the nblk scale bytes after them
// (the launcher checks 17*nblk % 16 == 0, i.e. hidden % 512 == 0).
template <int K, bool kEven, bool kPacked, bool kEager>
__global__ __launch_bounds__(kMxThreads) void k_dispatch_mxfp4(
    const u32x4* __restrict__ x, int64_t n_rows, int h16, int top_k,
    const uint32_t* __restrict__ restore, uint8_t* __restrict__ q, uint8_t* __restrict__ scales,
    uint32_t limit, RowSplit rs) {
  __shared__ uint32_t s_pos[K > 0 ? 1 : kMaxTopK];
  __shared__ int s_n;
  constexpr int KR = K > 0 ? K : 1;
  const int nblk = h16 / 4;
  const int64_t items = n_rows * rs.split;
  for (int64_t item = blockIdx.x; item < items; item += gridDim.x) {
    const int64_t t = rs.split == 1 ? item : item / rs.split;
    const int lo = int(item - t * rs.split) * rs.len;  // this workgroup's blocks [lo, hi)
    const int hi = min(nblk, lo + rs.len);
    const u32x4* src = x + t * h16;
    const int b0 = lo + int(threadIdx.x);
    static_assert(!kEager || K > 0, "eager loads need the positions in registers");
    u32x4 first[kEager ? 4 : 1];
    if constexpr (kEager) {
      if (b0 < hi) {
#pragma unroll
        for (int u = 0; u < 4; ++u) first[u] = load_vec<MOE_MXFP4_NT_LOAD>(src + 4 * b0 + u);
      }
    }
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
    for (int b = b0; n > 0 && b < hi; b += kMxThreads) {
      uint32_t w[16];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const u32x4 v = (kEager && b == b0) ? first[u] : load_vec<MOE_MXFP4_NT_LOAD>(src + 4 * b + u);
        w[4 * u + 0] = v.x;
        w[4 * u + 1] = v.y;
        w[4 * u + 2] = v.z;
        w[4 * u + 3] = v.w;
      }
      uint32_t amax = 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) amax = max(amax, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
      const int se = mx_scale_exponent<kEven>(amax);
      const float scale = pow2_f32(se);
      u32x4 pv;
      pv.x = e2m1_word(w + 0, scale);
      pv.y = e2m1_word(w + 4, scale);
      pv.z = e2m1_word(w + 8, scale);
      pv.w = e2m1_word(w + 12, scale);
      const uint8_t sbyte = uint8_t(se + 127);
      const int nj = K > 0 ? K : n;
#pragma unroll
      for (int j = 0; j < nj; ++j) {
        const uint32_t p32 = K > 0 ? pos[j] : s_pos[j];
        if (p32 == kSent) continue;
        const int64_t p = p32;
        if constexpr (kPacked) {
          uint8_t* row = q + p * (int64_t(nblk) * 17);  // 16 payload bytes + 1 scale byte per block
          store_vec<MOE_MXFP4_PACKED_NT_STORE>(reinterpret_cast<u32x4*>(row) + b, pv);
          row[int64_t(nblk) * 16 + b] = sbyte;
        } else {
          store_vec<MOE_MXFP4_NT_STORE>(reinterpret_cast<u32x4*>(q) + p * nblk + b, pv);
          scales[p * nblk + b] = sbyte;
        }
      }
    }
    if constexpr (K == 0) __syncthreads();  // s_pos is rewritten for the next token
  }
}

namespace {

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

template <int K>
struct LaunchMxfp4 {
  template <bool kEven, bool kPacked>
  static hipError_t go(const u32x4* x, int64_t n_rows, int h16, int top_k,
                       const uint32_t* restore, uint8_t* q, uint8_t* scales, uint32_t limit,
                       hipStream_t s) {
    const RowSplit rs = row_split(n_rows, h16 / 4, kMxThreads / 2);
    const double out_bytes = double(n_rows) * top_k * (h16 / 4) * 17.0;
    const dim3 grid(row_grid(n_rows * rs.split)), block(kMxThreads);
    if constexpr (K > 0) {
      if (out_bytes >= double(MOE_MXFP4_EAGER_MIN_BYTES) && out_bytes < double(MOE_MXFP4_EAGER_MAX_BYTES)) {
        hipLaunchKernelGGL((k_dispatch_mxfp4<K, kEven, kPacked, true>), grid, block, 0, s, x, n_rows,
                           h16, top_k, restore, q, scales, limit, rs);
        return hipGetLastError();
      }
    }
    hipLaunchKernelGGL((k_dispatch_mxfp4<K, kEven, kPacked, false>), grid, block, 0, s, x, n_rows, h16,
                       top_k, restore, q, scales, limit, rs);
    return hipGetLastError();
  }
  static hipError_t run(const u32x4* x, int64_t n_rows, int h16, int top_k, const uint32_t* restore,
                        uint8_t* q, uint8_t* scales, uint32_t limit, int mode, hipStream_t s) {
    switch (mode) {
      case 0: return go<false, false>(x, n_rows, h16, top_k, restore, q, scales, limit, s);
      case 1: return go<true, false>(x, n_rows, h16, top_k, restore, q, scales, limit, s);
      case 2: return go<false, true>(x, n_rows, h16, top_k, restore, q, scales, limit, s);
      default: return go<true, true>(x, n_rows, h16, top_k, restore, q, scales, limit, s);
    }
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

hipError_t launch_dispatch_mxfp4(const uint16_t* x, int64_t n_rows, int hidden, int top_k,
                                 const uint32_t* restore, uint8_t* q, uint8_t* scales,
                                 int64_t out_rows, bool even_scale, bool packed, hipStream_t s) {
  if (n_rows == 0) return hipSuccess;
  const int mode = (even_scale ? 1 : 0) | (packed ? 2 : 0);
  return by_top_k<LaunchMxfp4>(top_k, reinterpret_cast<const u32x4*>(x), n_rows, hidden / 8, top_k,
                               restore, q, scales, position_limit(out_rows), mode, s);
}

}  // namespace moe
