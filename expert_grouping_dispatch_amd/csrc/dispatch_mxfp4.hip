// Stage 3b: dispatch token rows into the expert-contiguous buffer as MXFP4
// ("Struct_ep_dispatch_async_mxfp4", execute: tokens travel as FP4 quants
// with their scales; Parameters dispatch_dtype, dispatch_scale_dtype).
// Each 32-element block of a token row is encoded once (E2M1 payload, one
// E8M0 scale byte) and written to every routed position of the token, so x
// is read once per token.  Two lane layouts, chosen by output size (measured
// on MI355X): one lane per block for outputs under MOE_MXFP4_QUAD_MIN_BYTES
// and any top_k (k_dispatch_mxfp4), four lanes per block with consecutive
// loads for larger outputs with top_k <= 8 (k_dispatch_mxfp4_quad).
#include "common.h"
#include "internal.h"
#include "rows.h"

namespace moe {

namespace {

// Lanes per workgroup of the one-lane-per-block kernel.
#ifndef MOE_MXFP4_THREADS
#define MOE_MXFP4_THREADS 256
#endif
// Outputs (payload and scales) of at least MOE_MXFP4_QUAD_MIN_BYTES with
// top_k <= 8 take the four-lanes-per-block kernel, whose workgroups have at
// most MOE_MXFP4_QUAD_THREADS lanes, each loading MOE_MXFP4_QUAD_UNITS
// 16-byte quarters of blocks per step.  It loads x non-temporally when x
// holds at least MOE_MXFP4_QUAD_NT_LOAD_MIN_BYTES, more than the 256 MB
// Infinity Cache keeps for the next reader.  Measured on MI355X with
// 7168-wide rows and top_k 8: on a 2.75 GB output (x 939 MB), one quarter
// per step and non-temporal loads take 0.48 ms in the pipeline against
// 0.53 ms with two quarters and plain loads (each change alone gains about
// half of that); non-temporal loads also win on x of 352 and 470 MB (2% and
// 3%) but lose on x of 176 and 235 MB (0.105 ms against 0.083 ms, 0.138 ms
// against 0.109 ms), which stays in that cache between calls.
#ifndef MOE_MXFP4_QUAD_MIN_BYTES
#define MOE_MXFP4_QUAD_MIN_BYTES (int64_t(256) << 20)
#endif
#ifndef MOE_MXFP4_QUAD_THREADS
#define MOE_MXFP4_QUAD_THREADS 512
#endif
#ifndef MOE_MXFP4_QUAD_UNITS
#define MOE_MXFP4_QUAD_UNITS 1
#endif
#ifndef MOE_MXFP4_QUAD_NT_LOAD_MIN_BYTES
#define MOE_MXFP4_QUAD_NT_LOAD_MIN_BYTES (int64_t(256) << 20)
#endif
// Cache policy of k_dispatch_mxfp4 (measured on MI355X): plain loads of x;
// for the separate payload rows (128-byte aligned), plain stores for outputs of
// [MOE_MXFP4_PLAIN_MIN_BYTES, MOE_MXFP4_PLAIN_MAX_BYTES), which the Infinity
// Cache absorbs (a 36 MB output's pipeline 2.5% faster), and the
// MOE_MXFP4_NT_STORE policy otherwise: non-temporal, since a 125 MB output
// then leaves the next kernel more dirty lines to drain (its pipeline 0.9%
// slower with plain stores), a 1.87 GB one took 4.5% longer, and the
// latency-bound small outputs gain nothing (the same time on 8 MB).
#ifndef MOE_MXFP4_NT_LOAD
#define MOE_MXFP4_NT_LOAD 0
#endif
#ifndef MOE_MXFP4_NT_STORE
#define MOE_MXFP4_NT_STORE 1
#endif
#ifndef MOE_MXFP4_PLAIN_MIN_BYTES
#define MOE_MXFP4_PLAIN_MIN_BYTES (int64_t(16) << 20)
#endif
#ifndef MOE_MXFP4_PLAIN_MAX_BYTES
#define MOE_MXFP4_PLAIN_MAX_BYTES (int64_t(64) << 20)
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
// faster on 3-30 MB outputs, which would only read more.
#ifndef MOE_MXFP4_EAGER_MIN_BYTES
#define MOE_MXFP4_EAGER_MIN_BYTES (int64_t(64) << 20)
#endif
#ifndef MOE_MXFP4_EAGER_MAX_BYTES
#define MOE_MXFP4_EAGER_MAX_BYTES (int64_t(256) << 20)
#endif
constexpr int kMxThreads = MOE_MXFP4_THREADS;
constexpr int kMxQuadThreads = MOE_MXFP4_QUAD_THREADS;
constexpr int kMxQuadUnits = MOE_MXFP4_QUAD_UNITS;
static_assert(kMxQuadThreads % 64 == 0 && kMxQuadThreads <= 1024, "whole waves, at most 1024 lanes");
static_assert(kMxQuadUnits >= 1 && kMxQuadUnits <= 16, "16-byte vectors per lane and step");

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
// maximum.  The pairs come in as plain 32-bit words: bit casts of a
// vector's elements taken in place were compiled to the first element's
// register.
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

// Largest 15-bit magnitude of the eight bf16 values of four 32-bit words.
__device__ __forceinline__ uint32_t words_amax(const uint32_t* w) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) m = max(m, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
  return m;
}

}  // namespace

// One lane per 32-element block: 4 x 16-byte loads, 16 bytes of payload and
// one scale byte per routed position.  K > 0: top_k == K, positions in
// scalar registers; K == 0: any top_k, positions compacted into LDS by wave
// 0.  kPacked: one row of 17*nblk bytes per slot, the 16*nblk payload bytes
// first and the nblk scale bytes after them (the launcher checks
// 17*nblk % 16 == 0, i.e. hidden % 512 == 0).  kEager (K > 0 only): each
// lane's first block of x is requested before the positions.  kNtStore:
// non-temporal payload stores (separate rows).
template <int K, bool kEven, bool kPacked, bool kEager, bool kNtStore>
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
      for (int u = 0; u < 4; ++u) amax = max(amax, words_amax(w + 4 * u));
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
          store_vec<kNtStore>(reinterpret_cast<u32x4*>(q) + p * nblk + b, pv);
          scales[p * nblk + b] = sbyte;
        }
      }
    }
    if constexpr (K == 0) __syncthreads();  // s_pos is rewritten for the next token
  }
}

// Four lanes per 32-element block, for top_k == K <= 8, one workgroup per
// token.  The workgroup's lanes form quads; in step u, lane r of quad m owns
// quarter r (8 elements, one 16-byte vector) of block u*lanes/4 + m, so
// every load instruction reads lanes*16 consecutive bytes of x.  The block
// maximum meets across the quad by DPP; each lane encodes its 8 elements
// into one 32-bit word of payload and stores it to each routed position
// (consecutive lanes write consecutive words); lane 0 of the quad stores the
// scale byte.  kPacked as in k_dispatch_mxfp4; kNtLoad: non-temporal loads
// of x.  The launcher makes `lanes` a multiple of 4, and a row is a whole
// number of blocks, so the four lanes of a quad are active together.
template <int K, bool kEven, bool kPacked, bool kNtLoad>
__global__ __launch_bounds__(kMxQuadThreads) void k_dispatch_mxfp4_quad(
    const u32x4* __restrict__ x, int h16, const uint32_t* __restrict__ restore,
    uint8_t* __restrict__ q, uint8_t* __restrict__ scales, uint32_t limit) {
  constexpr int U = kMxQuadUnits;
  const int lanes = blockDim.x, tid = threadIdx.x;
  const int64_t t = blockIdx.x;
  const int nblk = h16 / 4;
  uint32_t pos[K];
  float unused[K];
  uniform_slots<K, false>(restore, nullptr, t, limit, pos, unused);
  bool any = false;
#pragma unroll
  for (int j = 0; j < K; ++j) any |= pos[j] != kSent;
  if (!any) return;
  const u32x4* src = x + t * h16;
  const int64_t row_words = int64_t(nblk) * (kPacked ? 17 : 16) / 4;  // 32-bit words per output row
  for (int base = 0; base < h16; base += U * lanes) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int unit = base + u * lanes + tid;
      v[u] = unit < h16 ? load_vec<kNtLoad>(src + unit) : u32x4{0u, 0u, 0u, 0u};
    }
    uint32_t word[U], sbyte[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t w4[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
      const int se = mx_scale_exponent<kEven>(quad_max(words_amax(w4)));
      word[u] = e2m1_word(w4, pow2_f32(se));
      sbyte[u] = uint32_t(se + 127);
    }
#pragma unroll
    for (int j = 0; j < K; ++j) {
      if (pos[j] == kSent) continue;
      uint32_t* prow = reinterpret_cast<uint32_t*>(q) + int64_t(pos[j]) * row_words;
      uint8_t* srow = kPacked ? reinterpret_cast<uint8_t*>(prow) + int64_t(nblk) * 16 : scales + int64_t(pos[j]) * nblk;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int unit = base + u * lanes + tid;
        if (unit < h16) {
          if constexpr (kPacked ? MOE_MXFP4_PACKED_NT_STORE : MOE_MXFP4_NT_STORE)
            __builtin_nontemporal_store(word[u], prow + unit);
          else
            prow[unit] = word[u];
          if ((tid & 3) == 0) srow[unit / 4] = uint8_t(sbyte[u]);
        }
      }
    }
  }
}

namespace {

template <int K>
struct LaunchMxfp4 {
  template <bool kEven, bool kPacked>
  static hipError_t go(const u32x4* x, int64_t n_rows, int h16, int top_k,
                       const uint32_t* restore, uint8_t* q, uint8_t* scales, uint32_t limit,
                       hipStream_t s) {
    const double out_bytes = double(n_rows) * top_k * (h16 / 4) * 17.0;
    if constexpr (K > 0) {
      if (out_bytes >= double(MOE_MXFP4_QUAD_MIN_BYTES) && n_rows < (int64_t(1) << 31)) {
        // the fewest quads that cover the row in kMxQuadUnits steps, at most kMxQuadThreads lanes
        const int quads = (h16 / 4 + kMxQuadUnits - 1) / kMxQuadUnits;
        const dim3 grid{uint32_t(n_rows)}, block{uint32_t(min(4 * quads, kMxQuadThreads))};
        if (double(n_rows) * h16 * 16 >= double(MOE_MXFP4_QUAD_NT_LOAD_MIN_BYTES))
          hipLaunchKernelGGL((k_dispatch_mxfp4_quad<K, kEven, kPacked, true>), grid, block, 0, s, x, h16,
                             restore, q, scales, limit);
        else
          hipLaunchKernelGGL((k_dispatch_mxfp4_quad<K, kEven, kPacked, false>), grid, block, 0, s, x, h16,
                             restore, q, scales, limit);
        return hipGetLastError();
      }
    }
    const RowSplit rs = row_split(n_rows, h16 / 4, kMxThreads / 2);
    const dim3 grid(row_grid(n_rows * rs.split)), block(kMxThreads);
    const bool plain =
        out_bytes >= double(MOE_MXFP4_PLAIN_MIN_BYTES) && out_bytes < double(MOE_MXFP4_PLAIN_MAX_BYTES);
    constexpr bool kNt = MOE_MXFP4_NT_STORE != 0;
#define MOE_MXFP4_GO(EAGER, NT)                                                                     \
  hipLaunchKernelGGL((k_dispatch_mxfp4<K, kEven, kPacked, EAGER, NT>), grid, block, 0, s, x, n_rows, \
                     h16, top_k, restore, q, scales, limit, rs)
    if constexpr (K > 0) {
      if (out_bytes >= double(MOE_MXFP4_EAGER_MIN_BYTES) && out_bytes < double(MOE_MXFP4_EAGER_MAX_BYTES)) {
        if (plain) MOE_MXFP4_GO(true, false);
        else MOE_MXFP4_GO(true, kNt);
        return hipGetLastError();
      }
    }
    if (plain) MOE_MXFP4_GO(false, false);
    else MOE_MXFP4_GO(false, kNt);
#undef MOE_MXFP4_GO
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

hipError_t launch_dispatch_mxfp4(const uint16_t* x, int64_t n_rows, int hidden, int top_k,
                                 const uint32_t* restore, uint8_t* q, uint8_t* scales,
                                 int64_t out_rows, bool even_scale, bool packed, hipStream_t s) {
  if (n_rows == 0) return hipSuccess;
  const int mode = (even_scale ? 1 : 0) | (packed ? 2 : 0);
  return by_top_k<LaunchMxfp4>(top_k, reinterpret_cast<const u32x4*>(x), n_rows, hidden / 8, top_k,
                               restore, q, scales, position_limit(out_rows), mode, s);
}

}  // namespace moe
