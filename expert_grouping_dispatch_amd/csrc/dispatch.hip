// Stage 3: dispatch token rows into the expert-contiguous buffer, as bf16 or
// as MXFP4 ("Struct_ep_dispatch_async_mxfp4": input_tokens [num_tokens,
// hidden_size] go to the experts of topk_ids; FP4 quants travel with their
// scales).  Token-major: one workgroup per token (per part of the row when
// there are few rows) reads the row once and writes it to each of its routed
// positions, so x is read once per token instead of once per slot.
#include "common.h"
#include "internal.h"
#include "rows.h"

namespace moe {

namespace {

#ifndef MOE_DISPATCH_LOADS
#define MOE_DISPATCH_LOADS 4
#endif
#ifndef MOE_DISPATCH_THREADS
#define MOE_DISPATCH_THREADS 256
#endif
#ifndef MOE_MXFP4_THREADS
#define MOE_MXFP4_THREADS 256
#endif
// Cache policy (measured on MI355X: plain loads and stores for the bf16 row
// fan-out, plain loads and non-temporal stores for the separate MXFP4 payload
// rows, which are 128-byte aligned).
#ifndef MOE_DISPATCH_NT_LOAD
#define MOE_DISPATCH_NT_LOAD 0
#endif
#ifndef MOE_DISPATCH_NT_STORE
#define MOE_DISPATCH_NT_STORE 0
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
constexpr int kLoadsInFlight = MOE_DISPATCH_LOADS;  // 16-byte vectors each lane loads before storing
constexpr int kDispatchThreads = MOE_DISPATCH_THREADS;
constexpr int kMxThreads = MOE_MXFP4_THREADS;

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

// K > 0: top_k == K and the positions sit in scalar registers; K == 0: any
// top_k, positions compacted into LDS by wave 0.
template <int K>
__global__ __launch_bounds__(kDispatchThreads) void k_dispatch_bf16(
    const u32x4* __restrict__ x, int64_t n_rows, int h16, int top_k,
    const uint32_t* __restrict__ restore, u32x4* __restrict__ out, uint32_t limit, RowSplit rs) {
  __shared__ uint32_t s_pos[K > 0 ? 1 : kMaxTopK];
  __shared__ int s_n;
  constexpr int KR = K > 0 ? K : 1;
  const int64_t items = n_rows * rs.split;
  for (int64_t item = blockIdx.x; item < items; item += gridDim.x) {
    const int64_t t = rs.split == 1 ? item : item / rs.split;
    const int lo = int(item - t * rs.split) * rs.len;  // this workgroup's vectors [lo, hi)
    const int hi = min(h16, lo + rs.len);
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
    const u32x4* src = x + t * h16;
    for (int c0 = lo + int(threadIdx.x); n > 0 && c0 < hi; c0 += kDispatchThreads * kLoadsInFlight) {
      u32x4 v[kLoadsInFlight];
#pragma unroll
      for (int u = 0; u < kLoadsInFlight; ++u) {
        const int c = c0 + u * kDispatchThreads;
        if (c < hi) v[u] = load_vec<MOE_DISPATCH_NT_LOAD>(src + c);
      }
      const int nj = K > 0 ? K : n;
#pragma unroll
      for (int j = 0; j < nj; ++j) {
        const uint32_t p = K > 0 ? pos[j] : s_pos[j];
        if (p == kSent) continue;
        u32x4* dst = out + int64_t(p) * h16;
#pragma unroll
        for (int u = 0; u < kLoadsInFlight; ++u) {
          const int c = c0 + u * kDispatchThreads;
          if (c < hi) store_vec<MOE_DISPATCH_NT_STORE>(dst + c, v[u]);
        }
      }
    }
    if constexpr (K == 0) __syncthreads();  // s_pos is rewritten for the next token
  }
}

// One lane per 32-element block: 4 x 16-byte loads, 16 bytes of payload and
// one scale byte per routed position.  kPacked: one row of 17*nblk bytes per
// slot, the 16*nblk payload bytes first and the nblk scale bytes after them
// (the launcher checks 17*nblk % 16 == 0, i.e. hidden % 512 == 0).
template <int K, bool kEven, bool kPacked>
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
    const u32x4* src = x + t * h16;
    for (int b = lo + int(threadIdx.x); n > 0 && b < hi; b += kMxThreads) {
      uint32_t w[16];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const u32x4 v = load_vec<MOE_MXFP4_NT_LOAD>(src + 4 * b + u);
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
    const RowSplit rs = row_split(n_rows, h16, kDispatchThreads / 2);
    hipLaunchKernelGGL(k_dispatch_bf16<K>, dim3(row_grid(n_rows * rs.split)), dim3(kDispatchThreads),
                       0, s, x, n_rows, h16, top_k, restore, out, limit, rs);
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
    hipLaunchKernelGGL((k_dispatch_mxfp4<K, kEven, kPacked>), dim3(row_grid(n_rows * rs.split)),
                       dim3(kMxThreads), 0, s, x, n_rows, h16, top_k, restore, q, scales, limit, rs);
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
