// Stage 2: expert-grouped indices ("moe_create_indices": histogram the expert
// ids, scan the histogram into CSR offsets, scatter the slots).
//
// The pages' kernel is one CTA.  Here the slots are cut into chunks (of
// kIdxChunk slots, or half that for inputs up to kIdxSmallMaxSlots so that
// more workgroups share them); for S <= kIdxChunk one workgroup of the
// fewest whole waves that hold the slots does all three steps in one launch
// (k_index_one).  With at most 16 experts and few chunks, one launch of one
// workgroup per chunk (k_index_few) in which every workgroup counts all the
// slots itself.  Other inputs of more chunks take two launches, one
// workgroup per chunk:
//   up to kIdxSumMaxChunks chunks with a count table of at most
//   kIdxSumMaxEntries entries (every workload here), without waits:
//     k_index_count        LDS histogram -> one row of 16-bit counts;
//     k_index_scatter_sum  sums the whole table (totals -> bucket starts;
//                          rows before its chunk -> its offsets), chunk 0
//                          writes the CSR / active-expert / stats outputs,
//                          then the stable scatter;
//   larger inputs, where that table would be read too many times:
//     k_index_hist     per chunk (taken by ticket): LDS histogram, then a
//                      decoupled lookback over earlier chunks gives, per
//                      bucket, the number of slots in all earlier chunks; the
//                      chunk holding the last ticket also has the totals and
//                      writes the CSR / active-expert / stats outputs;
//     k_index_scatter  per chunk: stable ranks -> token_expert_order and
//                      restore_token_order.
// Stable ranks come from wave ballots and per-wave LDS counters.  The
// workspace layout does not depend on the call's shape (header, bucket
// starts, the count table at its largest, then the lookback words), and
// k_index_scatter zeroes every lookback word it has read, so between calls
// the word region holds zeros only and a later call of any shape finds no
// published word it did not write.  The count table is rewritten by every
// call that reads it.
// Bucket b < E is expert b; bucket E collects the unrouted slots, which land
// after every routed slot and fill token_expert_order[V, S) with sentinels.
// For the one-call mask + index entry point, the first kernel also counts the
// slots of padding rows as unrouted and writes -1 into them, so the scatter
// reads the masked map.
#include "common.h"
#include "internal.h"

namespace moe {

namespace {

// lookback word: [33:32] status (0 = not yet published), [31:0] count
constexpr uint64_t kFlagAggregate = uint64_t(1) << 32;  // count of this chunk only
constexpr uint64_t kFlagPrefix = uint64_t(2) << 32;     // count of chunks [0, c]
constexpr uint32_t kSpinLimit = 1u << 20;
#ifndef MOE_LOOKBACK_WINDOW
#define MOE_LOOKBACK_WINDOW 4
#endif
constexpr int kLookbackWindow = MOE_LOOKBACK_WINDOW;
// Up to this many buckets (5 per lane), wave 0 alone scans the bucket
// totals and writes the CSR outputs, with no barrier, while the other waves
// go on; more buckets take the block-wide scan.
#ifndef MOE_IDX_WAVE_FINALIZE_MAX_BUCKETS
#define MOE_IDX_WAVE_FINALIZE_MAX_BUCKETS 320
#endif
constexpr int kWaveFinalizeMaxBuckets = MOE_IDX_WAVE_FINALIZE_MAX_BUCKETS;
constexpr int kWaveFinalizeIpt = (kWaveFinalizeMaxBuckets + kWave - 1) / kWave;  // buckets per lane
static_assert(kWaveFinalizeMaxBuckets >= 1 && kWaveFinalizeMaxBuckets <= MOE_MAX_BUCKETS,
              "the one-wave scan covers at most every bucket");
static_assert(MOE_IDX_FEW_MAX_EXPERTS + 1 <= kWave, "the few-expert pass scans one bucket per lane");

size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

__device__ __forceinline__ uint32_t bucket_of(int32_t id, uint32_t n_experts) {
  return uint32_t(id) < n_experts ? uint32_t(id) : n_experts;
}

__device__ __forceinline__ uint32_t bucket_of(int64_t id, uint32_t n_experts) {
  return uint64_t(id) < uint64_t(n_experts) ? uint32_t(id) : n_experts;
}

__device__ __forceinline__ bool is_leader(uint64_t peers) {
  return peers != 0 && __builtin_ctzll(peers) == int(__lane_id());
}

// First slot of the padding rows to mask (n_slots when nothing is masked):
// the boundary count - tp_rank * n_rows, clamped to [0, n_rows], in 64 bits.
__device__ __forceinline__ int64_t pad_begin(const PadMask& pad, int64_t n_slots) {
  if (pad.count == nullptr) return n_slots;
  const int64_t n_rows = n_slots / pad.top_k;
  int64_t first = int64_t(*pad.count) - int64_t(pad.tp_rank) * n_rows;
  first = first < 0 ? 0 : (first > n_rows ? n_rows : first);
  return first * pad.top_k;
}

// The ids of R slots, loaded before any is used so that the loads of all
// rounds are in flight together.  A lane past the last slot loads the last
// slot again (in bounds) and its value is never used.  Only the
// one-workgroup pass can have no slots (kMayBeEmpty): then nothing is loaded.
// Elsewhere the loads take no branch, which would make each one wait.
template <bool kMayBeEmpty, int R, typename IdT>
__device__ __forceinline__ void load_ids(const IdT* ids, int64_t n_slots, int64_t first,
                                         int64_t stride, IdT (&id)[R]) {
  if (kMayBeEmpty && n_slots == 0) {
#pragma unroll
    for (int r = 0; r < R; ++r) id[r] = IdT(0);
    return;
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t i = first + r * stride;
    id[r] = ids[i < n_slots ? i : n_slots - 1];
  }
}

// Bucket of slot i with id `id`; slots at or past pad_from are padding:
// unrouted, and set to -1 through wmap (the same map, writable) when masking.
// Each slot is read and written by the same thread, and no other workgroup of
// the kernel reads it.
template <typename IdT>
__device__ __forceinline__ uint32_t slot_key(IdT id, IdT* wmap, int64_t i, int64_t pad_from,
                                             uint32_t n_experts) {
  if (i < pad_from) return bucket_of(id, n_experts);
  if (wmap != nullptr) wmap[i] = IdT(-1);
  return n_experts;
}

// Count the chunk's slots per bucket into hist[0..E] (LDS, zeroed by caller).
// Only totals are needed here, so plain LDS atomics do.
template <int R, int T, typename IdT>
__device__ void chunk_histogram(const IdT* ids, IdT* wmap, int64_t n_slots, int64_t begin,
                                uint32_t n_experts, uint32_t* hist, int64_t pad_from) {
  const int tid = threadIdx.x;
  IdT id[R];
  load_ids<false, R>(ids, n_slots, begin + tid, T, id);
  uint32_t key[R];
  bool valid[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t i = begin + int64_t(r) * T + tid;
    valid[r] = i < n_slots;
    key[r] = valid[r] ? slot_key(id[r], wmap, i, pad_from, n_experts) : 0u;
  }
#pragma unroll
  for (int r = 0; r < R; ++r)
    if (valid[r]) atomicAdd(&hist[key[r]], 1u);
}

// One wave's slots of a chunk of R rounds: wave w owns the R*64 consecutive
// slots starting at begin + w*R*64, so (wave, round, lane) order is
// ascending slot index.  Keys and peer masks stay in registers between the
// counting pass and the scatter pass.
template <int R>
struct WaveTile {
  uint32_t key[R];
  bool valid[R];
  uint64_t peers[R];
  int64_t wbegin;
};

// The ids of the wave's slots of a chunk starting at `begin`.
template <bool kMayBeEmpty, int R, typename IdT>
__device__ __forceinline__ void wave_load_ids(const IdT* ids, int64_t n_slots, int64_t begin,
                                              IdT (&id)[R]) {
  const int wave = threadIdx.x / kWave;
  load_ids<kMayBeEmpty, R>(ids, n_slots, begin + int64_t(wave) * R * kWave + __lane_id(), kWave, id);
}

// The tile's keys from the ids wave_load_ids loaded (the keys of padding
// slots are the unrouted bucket; with wmap given, those slots are set to -1).
template <int R, typename IdT>
__device__ __forceinline__ void wave_keys(const IdT (&id)[R], IdT* wmap, int64_t n_slots,
                                          int64_t begin, uint32_t n_experts, WaveTile<R>& tile,
                                          int64_t pad_from) {
  const int lane = __lane_id(), wave = threadIdx.x / kWave;
  tile.wbegin = begin + int64_t(wave) * R * kWave;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t i = tile.wbegin + r * kWave + lane;
    tile.valid[r] = i < n_slots;
    tile.key[r] = tile.valid[r] ? slot_key(id[r], wmap, i, pad_from, n_experts) : 0u;
  }
}

// Count the tile's keys per bucket into the wave's own LDS row
// whist[wave][0..E] (only this wave touches the row; no atomics).
template <int R>
__device__ __forceinline__ void wave_count_keys(uint32_t n_experts, int nbits, uint32_t* whist,
                                                WaveTile<R>& tile) {
  const int lane = __lane_id(), wave = threadIdx.x / kWave;
  const int nb = int(n_experts) + 1;
  uint32_t* my = whist + wave * nb;
  for (int b = lane; b < nb; b += kWave) my[b] = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    tile.peers[r] = match_peers(tile.key[r], nbits, tile.valid[r]);
    if (tile.valid[r] && is_leader(tile.peers[r])) my[tile.key[r]] += uint32_t(__popcll(tile.peers[r]));
  }
}

template <bool kMayBeEmpty, int R, typename IdT>
__device__ void wave_counts(const IdT* ids, IdT* wmap, int64_t n_slots, int64_t begin,
                            uint32_t n_experts, int nbits, uint32_t* whist, WaveTile<R>& tile,
                            int64_t pad_from) {
  IdT id[R];
  wave_load_ids<kMayBeEmpty>(ids, n_slots, begin, id);
  wave_keys(id, wmap, n_slots, begin, n_experts, tile, pad_from);
  wave_count_keys(n_experts, nbits, whist, tile);
}

// Stable scatter after wave_counts and a barrier.  off[b] (LDS) = position
// of the chunk's first slot of bucket b, or with kFromEnd the position just
// past its last one.  Turns whist into per-wave running starts (exclusive
// prefix over waves seeded with the chunk's start), then each slot's position
// is its wave's running start plus its rank among lower peer lanes.
template <bool kFromEnd, int R, int T>
__device__ void wave_scatter(const WaveTile<R>& tile, uint32_t n_experts, const uint32_t* off,
                             uint32_t* whist, uint32_t* __restrict__ teo,
                             uint32_t* __restrict__ restore, int64_t n_slots) {
  const int tid = threadIdx.x, lane = __lane_id(), wave = tid / kWave;
  const int nb = int(n_experts) + 1;
  constexpr int kWaves = T / kWave;
  for (int b = tid; b < nb; b += T) {
    uint32_t run = off[b];
    if (kFromEnd)
      for (int w = 0; w < kWaves; ++w) run -= whist[w * nb + b];
    for (int w = 0; w < kWaves; ++w) {
      const uint32_t c = whist[w * nb + b];
      whist[w * nb + b] = run;
      run += c;
    }
  }
  __syncthreads();
  uint32_t* my = whist + wave * nb;
  const uint64_t below = lanes_below();
#pragma unroll
  for (int r = 0; r < R; ++r) {
    uint32_t pos = 0;
    if (tile.valid[r]) pos = my[tile.key[r]] + uint32_t(__popcll(tile.peers[r] & below));
    if (tile.valid[r] && is_leader(tile.peers[r])) my[tile.key[r]] += uint32_t(__popcll(tile.peers[r]));
    if (tile.valid[r]) {
      const uint32_t i = uint32_t(tile.wbegin + r * kWave + lane);
      const bool routed = tile.key[r] < n_experts;
      restore[i] = routed ? pos : kSent;
      // positions are < n_slots whenever the workspace was used as documented;
      // the check keeps a misused one from writing out of bounds
      if (int64_t(pos) < n_slots) teo[pos] = routed ? i : kSent;
    }
  }
}

// Block-wide: from per-bucket totals tot[0..E] (LDS) write the bucket starts
// base[0..E] (exclusive scan, base[E] = V) and, when `outputs` is set, the
// compacted CSR outputs; with soff given, also the aligned offsets
// (exclusive scan over active experts of their counts rounded up to `align`);
// with add_to given, add_to[b] += base[b] as well.  T = kWave: called by
// wave 0 alone, with no barrier, so that the other waves can go on.  Each
// lane owns ipt = ceil((E+1)/T) consecutive buckets.  kMaxIpt > 0 bounds ipt
// at compile time (a caller that passes less than the default guarantees
// fewer buckets), and a lane's LDS reads are then issued together instead of
// one after another; kMaxIpt = 0 keeps a loop over ipt, the default beyond 8
// buckets a lane, where the unrolled form measured slower (1024 experts over
// 64 lanes: 12.8 against 12.0 us).
template <int T, int kMaxIpt = ((MOE_MAX_BUCKETS + T - 1) / T <= 8 ? (MOE_MAX_BUCKETS + T - 1) / T : 0)>
__device__ void finalize_counts(const uint32_t* tot, uint32_t n_experts, uint32_t* base,
                                uint32_t* __restrict__ esi, int32_t* __restrict__ expert_ids,
                                uint32_t* __restrict__ stats, uint32_t* __restrict__ soff,
                                uint32_t align, bool outputs = true, uint32_t* add_to = nullptr) {
  constexpr int kWaves = T / kWave;
  __shared__ uint32_t part[kWaves > 1 ? 4 * kWaves : 1];
  const int tid = threadIdx.x, lane = __lane_id(), wave = tid / kWave;
  const int nb = int(n_experts) + 1;
  const int ipt = (nb + T - 1) / T;  // <= kMaxIpt
  const int b0 = tid * ipt;
  const bool want_soff = soff != nullptr;
  constexpr int kV = kMaxIpt > 0 ? kMaxIpt : 1;
  uint32_t v[kV];  // kMaxIpt > 0: the lane's bucket totals, 0 past its buckets
  uint32_t s_tot = 0, s_act = 0, s_max = 0, s_al = 0;
  auto add_bucket = [&](int b, uint32_t x) {
    s_tot += x;
    if (b < int(n_experts) && x > 0) {
      s_act += 1u;
      s_max = max(s_max, x);
      if (want_soff) s_al += (x + align - 1) / align * align;
    }
  };
  if constexpr (kMaxIpt > 0) {
    // every read is issued (at a clamped address) so that none waits behind a branch
#pragma unroll
    for (int q = 0; q < kMaxIpt; ++q) {
      const uint32_t x = tot[min(b0 + q, nb - 1)];
      v[q] = (q < ipt && b0 + q < nb) ? x : 0u;
    }
#pragma unroll
    for (int q = 0; q < kMaxIpt; ++q) add_bucket(b0 + q, v[q]);
  } else {
    for (int q = 0; q < ipt; ++q)
      if (b0 + q < nb) add_bucket(b0 + q, tot[b0 + q]);
  }
  const uint32_t in_tot = wave_inclusive_sum(s_tot);
  const uint32_t in_act = wave_inclusive_sum(s_act);
  const uint32_t in_al = wave_inclusive_sum(s_al);
  const uint32_t w_max = wave_max(s_max);
  uint32_t p_tot = in_tot - s_tot, p_act = in_act - s_act, p_al = in_al - s_al;
  uint32_t all_tot = 0, all_act = 0, all_max = 0, all_al = 0;
  if constexpr (kWaves == 1) {
    all_tot = __builtin_amdgcn_readlane(in_tot, kWave - 1);
    all_act = __builtin_amdgcn_readlane(in_act, kWave - 1);
    all_max = w_max;
    all_al = __builtin_amdgcn_readlane(in_al, kWave - 1);
  } else {
    if (lane == kWave - 1) {
      part[wave] = in_tot;
      part[kWaves + wave] = in_act;
      part[2 * kWaves + wave] = w_max;
      part[3 * kWaves + wave] = in_al;
    }
    __syncthreads();
    for (int w = 0; w < kWaves; ++w) {
      if (w < wave) {
        p_tot += part[w];
        p_act += part[kWaves + w];
        p_al += part[3 * kWaves + w];
      }
      all_tot += part[w];
      all_act += part[kWaves + w];
      all_max = max(all_max, part[2 * kWaves + w]);
      all_al += part[3 * kWaves + w];
    }
  }
  // bucket b's start, its offsets and (chunk 0) its CSR entry; prev is add_to[b]
  auto place_bucket = [&](int b, uint32_t x, uint32_t prev) {
    base[b] = p_tot;
    if (add_to != nullptr) add_to[b] = prev + p_tot;
    if (outputs && b < int(n_experts) && x > 0) {
      expert_ids[p_act] = b;
      esi[p_act] = p_tot;
      if (want_soff) {
        soff[p_act] = p_al;
        p_al += (x + align - 1) / align * align;
      }
      ++p_act;
    }
    p_tot += x;
  };
  if constexpr (kMaxIpt > 0) {
    uint32_t prev[kMaxIpt];
#pragma unroll
    for (int q = 0; q < kMaxIpt; ++q) prev[q] = add_to != nullptr ? add_to[min(b0 + q, nb - 1)] : 0u;
#pragma unroll
    for (int q = 0; q < kMaxIpt; ++q)
      if (q < ipt && b0 + q < nb) place_bucket(b0 + q, v[q], prev[q]);
  } else {
    for (int q = 0; q < ipt; ++q) {
      const int b = b0 + q;
      if (b < nb) place_bucket(b, tot[b], add_to != nullptr ? add_to[b] : 0u);
    }
  }
  if (!outputs) return;
  const uint32_t n_routed = all_tot - tot[n_experts];
  for (uint32_t j = all_act + tid; j < n_experts; j += T) expert_ids[j] = -1;
  for (uint32_t j = all_act + tid; j <= n_experts; j += T) {
    esi[j] = n_routed;
    if (want_soff) soff[j] = all_al;
  }
  if (tid == 0) {
    stats[0] = all_max;
    stats[1] = all_act;
  }
}

// Number of slots of bucket b in chunks [0, c): walk back over earlier chunks'
// words, kLookbackWindow at a time, adding per-chunk counts until a chunk
// that already published its inclusive prefix.  Every earlier chunk is held
// by a workgroup that took its ticket first and publishes its own count
// without waiting, so the wait ends; kSpinLimit is a backstop that records an
// error instead of spinning forever.
__device__ uint32_t lookback(const uint64_t* flags, int64_t c, int nb, int b, uint32_t* err) {
  uint32_t excl = 0;
  int64_t cc = c - 1;
  uint32_t spins = 0;
  while (true) {
    uint64_t f[kLookbackWindow];
#pragma unroll
    for (int w = 0; w < kLookbackWindow; ++w)
      f[w] = (cc - w >= 0) ? agent_load_u64(&flags[(cc - w) * nb + b]) : kFlagPrefix;
    int used = 0;
    bool done = false;
#pragma unroll
    for (int w = 0; w < kLookbackWindow; ++w) {
      if (done || used < w) continue;
      const uint32_t st = uint32_t(f[w] >> 32) & 3u;
      if (st == 0) continue;  // not yet published
      excl += uint32_t(f[w]);
      used = w + 1;
      if (st == 2u) done = true;
    }
    if (done) return excl;
    cc -= used;
    if (used == 0 && ++spins > kSpinLimit) {
      atomicOr(err, 1u);
      return excl;
    }
  }
}

}  // namespace

// Inputs of up to R * T slots: one workgroup of T lanes counts per wave,
// totals the counts, scans them and scatters, in one launch.
template <typename IdT, int R, int T>
__global__ __launch_bounds__(T) void k_index_one(
    const IdT* ids, int64_t n_slots, uint32_t n_experts, int nbits, uint32_t* __restrict__ esi,
    int32_t* __restrict__ expert_ids, uint32_t* __restrict__ stats, uint32_t* __restrict__ soff,
    uint32_t align, uint32_t* __restrict__ teo, uint32_t* __restrict__ restore, PadMask pad,
    IdT* wmap) {
  extern __shared__ uint32_t lds[];
  constexpr int kWaves = T / kWave;
  const int nb = int(n_experts) + 1;
  uint32_t* hist = lds;
  uint32_t* base = lds + nb;
  uint32_t* whist = lds + 2 * nb;
  WaveTile<R> tile;
  wave_counts<true>(ids, wmap, n_slots, 0, n_experts, nbits, whist, tile, pad_begin(pad, n_slots));
  __syncthreads();
  for (int b = threadIdx.x; b < nb; b += T) {
    uint32_t t = 0;
    for (int w = 0; w < kWaves; ++w) t += whist[w * nb + b];
    hist[b] = t;
  }
  __syncthreads();
  if (nb <= kWaveFinalizeMaxBuckets) {
    if (threadIdx.x < kWave)
      finalize_counts<kWave, kWaveFinalizeIpt>(hist, n_experts, base, esi, expert_ids, stats, soff, align);
  } else {
    finalize_counts<T>(hist, n_experts, base, esi, expert_ids, stats, soff, align);
  }
  __syncthreads();
  wave_scatter<false, R, T>(tile, n_experts, base, whist, teo, restore, n_slots);
}

// Chunks of R rounds of kIdxThreads slots: histogram + lookback + (last
// ticket) CSR outputs; the scatter follows in k_index_scatter.
template <typename IdT, int R>
__global__ __launch_bounds__(kIdxThreads) void k_index_hist(
    const IdT* ids, int64_t n_slots, uint32_t n_experts, int /*nbits*/,
    int64_t n_chunks, IndexWorkspace ws, uint32_t* __restrict__ esi,
    int32_t* __restrict__ expert_ids, uint32_t* __restrict__ stats, uint32_t* __restrict__ soff,
    uint32_t align, PadMask pad, IdT* wmap) {
  extern __shared__ uint32_t lds[];
  __shared__ int64_t s_chunk;
  const int nb = int(n_experts) + 1;
  const int tid = threadIdx.x;
  uint32_t* hist = lds;

  if (tid == 0) {
    s_chunk = int64_t(__hip_atomic_fetch_add(ws.ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  }
  for (int b = tid; b < nb; b += kIdxThreads) hist[b] = 0;
  __syncthreads();
  const int64_t c = s_chunk;
  if (c >= n_chunks) {  // only a workspace that was not zero-filled hands out such a ticket
    if (tid == 0) atomicOr(ws.err, 2u);
    return;
  }
  chunk_histogram<R, kIdxThreads>(ids, wmap, n_slots, c * (int64_t(R) * kIdxThreads), n_experts, hist,
                     pad_begin(pad, n_slots));
  __syncthreads();

  for (int b = tid; b < nb; b += kIdxThreads) {
    const uint32_t local = hist[b];
    uint64_t* word = &ws.flags[c * nb + b];
    uint32_t excl = 0;
    if (c == 0) {
      agent_store_u64(word, kFlagPrefix | local);
    } else {
      agent_store_u64(word, kFlagAggregate | local);
      excl = lookback(ws.flags, c, nb, b, ws.err);
      agent_store_u64(word, kFlagPrefix | (excl + local));
    }
    hist[b] = excl + local;
  }
  __syncthreads();

  if (c == n_chunks - 1) {
    finalize_counts<kIdxThreads>(hist, n_experts, ws.base, esi, expert_ids, stats, soff, align);
    if (tid == 0)  // every ticket of this call is taken: reset for the next call
      __hip_atomic_store(ws.ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <typename IdT, int R>
__global__ __launch_bounds__(kIdxThreads) void k_index_scatter(
    const IdT* __restrict__ ids, int64_t n_slots, uint32_t n_experts, int nbits,
    IndexWorkspace ws, uint32_t* __restrict__ teo, uint32_t* __restrict__ restore) {
  extern __shared__ uint32_t lds[];
  const int nb = int(n_experts) + 1;
  const int64_t c = blockIdx.x;
  uint32_t* off = lds;
  // Start the offset loads before the key work so both are in flight
  // together.  The chunk's word holds the slots of bucket b in chunks [0, c];
  // base + that count is the end of the chunk's run of bucket b.  The word is
  // then zeroed for the next call (the previous kernel wrote it; nothing else
  // reads it).
  constexpr int kMaxPerThread = (MOE_MAX_BUCKETS + kIdxThreads - 1) / kIdxThreads;
  uint32_t offv[kMaxPerThread];
#pragma unroll
  for (int q = 0; q < kMaxPerThread; ++q) {
    const int b = threadIdx.x + q * kIdxThreads;
    offv[q] = b < nb ? ws.base[b] + uint32_t(ws.flags[c * nb + b]) : 0u;
  }
#pragma unroll
  for (int q = 0; q < kMaxPerThread; ++q) {
    const int b = threadIdx.x + q * kIdxThreads;
    if (b < nb) ws.flags[c * nb + b] = 0u;
  }
  WaveTile<R> tile;
  // the map was masked by k_index_hist, so it is read as it is now
  wave_counts<false>(ids, static_cast<IdT*>(nullptr), n_slots, c * (int64_t(R) * kIdxThreads), n_experts,
              nbits, lds + nb, tile, n_slots);
#pragma unroll
  for (int q = 0; q < kMaxPerThread; ++q) {
    const int b = threadIdx.x + q * kIdxThreads;
    if (b < nb) off[b] = offv[q];
  }
  __syncthreads();
  wave_scatter<true, R, kIdxThreads>(tile, n_experts, off, lds + nb, teo, restore, n_slots);
}

// Wait-free path for up to kIdxSumMaxChunks chunks.  k_index_count writes
// each chunk's slot count per bucket as one row of the count table (16-bit
// counts, rows of E+1 padded to a multiple of 8, so that a row is whole
// 16-byte vectors).  Every k_index_scatter_sum workgroup then reads the whole
// table: the column sums over all rows are the bucket totals (their scan
// gives the bucket starts), and the sums over the rows before its chunk give
// the chunk's offset inside each bucket.  No workgroup waits on another.
template <typename IdT, int R>
__global__ __launch_bounds__(kIdxThreads) void k_index_count(
    const IdT* ids, int64_t n_slots, uint32_t n_experts, uint16_t* __restrict__ counts, PadMask pad,
    IdT* wmap) {
  extern __shared__ uint32_t lds[];
  const int nb = int(n_experts) + 1, nbp = (nb + 7) & ~7;
  const int c = blockIdx.x;
  for (int b = threadIdx.x; b < nb; b += kIdxThreads) lds[b] = 0;
  __syncthreads();
  chunk_histogram<R, kIdxThreads>(ids, wmap, n_slots, int64_t(c) * (R * kIdxThreads), n_experts, lds,
                                  pad_begin(pad, n_slots));
  __syncthreads();
  uint16_t* row = counts + int64_t(c) * nbp;
  for (int b = threadIdx.x; b < nbp; b += kIdxThreads) row[b] = uint16_t(b < nb ? lds[b] : 0u);
}

// Column sums at vector q of rows r, r + step, ... < n_rows of the count
// table (16-byte vectors of eight 16-bit counts, `nw` vectors per row), B
// rows at a time: all B loads are issued before the first is used.  `pre`
// takes the rows before `before`.  Returns the first row not summed.
template <int B>
__device__ __forceinline__ int sum_rows(const u32x4* __restrict__ rows, int r, int step, int n_rows,
                                        int nw, int q, int before, uint32_t (&tot)[8],
                                        uint32_t (&pre)[8]) {
  for (; r + (B - 1) * step < n_rows; r += B * step) {
    u32x4 v[B];
#pragma unroll
    for (int u = 0; u < B; ++u) v[u] = rows[int64_t(r + u * step) * nw + q];
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
      const bool earlier = r + u * step < before;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        tot[2 * k] += w[k] & 0xFFFFu;
        tot[2 * k + 1] += w[k] >> 16;
        if (earlier) {
          pre[2 * k] += w[k] & 0xFFFFu;
          pre[2 * k + 1] += w[k] >> 16;
        }
      }
    }
  }
  return r;
}

template <typename IdT, int R>
__global__ __launch_bounds__(kIdxThreads) void k_index_scatter_sum(
    const IdT* __restrict__ ids, int64_t n_slots, uint32_t n_experts, int nbits, int n_chunks,
    const u32x4* __restrict__ rows, uint32_t* __restrict__ esi, int32_t* __restrict__ expert_ids,
    uint32_t* __restrict__ stats, uint32_t* __restrict__ soff, uint32_t align,
    uint32_t* __restrict__ teo, uint32_t* __restrict__ restore) {
  extern __shared__ uint32_t lds[];
  const int nb = int(n_experts) + 1, nbp = (nb + 7) & ~7;
  const int nw = nbp / 8;                                  // 16-byte vectors per row
  const int nwr = (nw + kWave - 1) / kWave * kWave;
  const int slices = kIdxThreads / nwr;                    // >= 1: nw <= 129
  const int c = blockIdx.x;
  uint32_t* tot = lds;                                     // [nbp] totals
  uint32_t* off = tot + nbp;                               // [nbp] earlier chunks, then start
  uint32_t* base = off + nbp;                              // [nb]  bucket starts
  uint32_t* whist = base + nb;                             // [waves][nb]

  // the ids' loads go out first and land while the table is summed
  const int64_t begin = int64_t(c) * (R * kIdxThreads);
  IdT id[R];
  wave_load_ids<false>(ids, n_slots, begin, id);
  for (int b = threadIdx.x; b < 2 * nbp; b += kIdxThreads) tot[b] = 0;  // tot and off
  __syncthreads();

  // lane q of slice s sums vector q over rows s, s + slices, ...
  const int slice = threadIdx.x / nwr, q = threadIdx.x - slice * nwr;
  if (slice < slices && q < nw) {
    uint32_t t[8] = {}, e[8] = {};
    // batches of 16 rows, then at most one each of 8, 4, 2 and 1
    int r = sum_rows<16>(rows, slice, slices, n_chunks, nw, q, c, t, e);
    r = sum_rows<8>(rows, r, slices, n_chunks, nw, q, c, t, e);
    r = sum_rows<4>(rows, r, slices, n_chunks, nw, q, c, t, e);
    r = sum_rows<2>(rows, r, slices, n_chunks, nw, q, c, t, e);
    sum_rows<1>(rows, r, slices, n_chunks, nw, q, c, t, e);
    // the slices' sums meet in LDS (returnless atomic adds)
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      atomicAdd(&tot[8 * q + k], t[k]);
      atomicAdd(&off[8 * q + k], e[k]);
    }
  }
  __syncthreads();
  // every workgroup scans the totals for the bucket starts (chunk 0 also
  // writes the CSR outputs) and adds them to its offsets; with few enough
  // buckets wave 0 does it alone while the other waves rank their keys
  if (nb <= kWaveFinalizeMaxBuckets) {
    if (threadIdx.x < kWave)
      finalize_counts<kWave, kWaveFinalizeIpt>(tot, n_experts, base, esi, expert_ids, stats, soff, align, c == 0,
                                               off);
  } else {
    finalize_counts<kIdxThreads>(tot, n_experts, base, esi, expert_ids, stats, soff, align, c == 0, off);
  }
  WaveTile<R> tile;
  wave_keys(id, static_cast<IdT*>(nullptr), n_slots, begin, n_experts, tile, n_slots);
  wave_count_keys(n_experts, nbits, whist, tile);
  __syncthreads();
  wave_scatter<false, R, kIdxThreads>(tile, n_experts, off, whist, teo, restore, n_slots);
}

// Few experts (E <= NB, NB = 8 or 16) and 2 to J chunk rounds: one launch,
// no workspace.  Every chunk workgroup counts all the slots itself, which
// must then cost only a few vector instructions per slot: each lane adds
// 1 << 8e into a 64-bit word per 8 experts (byte e counts expert e), and a
// wave sums its words once at the end.  Scalar per-expert ballot counts were
// tried first: the scalar unit, shared by the CU's 16 waves, then bounded the
// kernel.  Wave w takes round r of chunk q as its group j = q*R + r, so
// groups j < c*R lie in the chunks before chunk c.  Only routed slots are
// counted; the unrouted bucket gets what they leave, of all slots (totals)
// and of the c*R*kIdxThreads slots before the chunk (its offset).  The
// chunk's own ids are loaded once more in the layout of the scatter.  With
// at most 17 buckets, wave 0 alone scans the totals into the chunk's starts
// (and in chunk 0 writes the CSR outputs) while the other waves rank their
// keys; then the scatter follows as in k_index_scatter_sum.  Padding slots
// (the one-call mask + index) are unrouted everywhere; only the owning chunk
// writes -1 into them, and the other workgroups, which may read either
// value, never look at it.  n_slots < 2^31 here, so slot indices are 32-bit.
template <typename IdT, int R, int NB, int J>
__global__ __launch_bounds__(kIdxThreads) void k_index_few(
    const IdT* ids, int64_t n_slots, uint32_t n_experts, int nbits, int n_chunks,
    uint32_t* __restrict__ esi, int32_t* __restrict__ expert_ids, uint32_t* __restrict__ stats,
    uint32_t* __restrict__ soff, uint32_t align, uint32_t* __restrict__ teo,
    uint32_t* __restrict__ restore, PadMask pad, IdT* wmap) {
  extern __shared__ uint32_t lds[];
  __shared__ uint32_t wcount[2][kIdxWaves][NB / 2];  // per wave, packed: all slots, slots before the chunk
  constexpr uint32_t kChunkSlots = uint32_t(R) * kIdxThreads;
  const int nb = int(n_experts) + 1;
  const int c = blockIdx.x;
  const int tid = threadIdx.x, lane = __lane_id(), wave = tid / kWave;
  uint32_t* tot = lds;          // [nb] slots of each bucket in all chunks
  uint32_t* off = tot + nb;     // [nb] in the chunks before this one, then this chunk's start
  uint32_t* base = off + nb;    // [nb] bucket starts
  uint32_t* whist = base + nb;  // [waves][nb]
  const int64_t pad_from = pad_begin(pad, n_slots);
  const uint32_t n32 = uint32_t(n_slots), pad32 = uint32_t(pad_from);
  const int64_t begin = int64_t(c) * kChunkSlots;
  IdT own[R];
  wave_load_ids<false>(ids, n_slots, begin, own);
  // all J groups' ids requested together through a bounds-checked buffer
  // resource, so that no load needs a clamp: a slot past the last reads 0
  // and is not counted.  Slot of group j: first(j) + lane_base.  64-bit ids
  // are reduced to 32 bits at once (kSent when not an expert), so that 32
  // groups of them need no more registers than 32-bit ones.
  // last resource word 0x00020000: 32-bit data format (bits 15-18 = 4), no
  // swizzle, no index stride; a raw load at or past the size returns 0
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<IdT*>(ids), 0, int(n32 * sizeof(IdT)), 0x00020000);
  const uint32_t lane_base = uint32_t(wave * R) * kWave + lane;
  uint32_t idv[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const uint32_t first = uint32_t(j / R) * kChunkSlots + uint32_t(j % R) * kWave;
    const int voff = int((first + lane_base) * sizeof(IdT));
    if constexpr (sizeof(IdT) == 4) {
      idv[j] = __builtin_amdgcn_raw_buffer_load_b32(rsrc, voff, 0, 0);
    } else {
      const uint64_t id = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(rsrc, voff, 0, 0));
      idv[j] = id < uint64_t(n_experts) ? uint32_t(id) : kSent;
    }
  }
  const int n_groups = n_chunks * R, g_own = c * R;
  // per lane, byte e of cnt[h] counts the lane's slots of expert 8h + e (at
  // most J <= 32 per byte); snap holds the counts of the groups before the
  // chunk, a prefix of the loop.  A slot counts when it lies before pad32
  // (padding and past the last slot do not) and its id is an expert.
  constexpr int H = NB / 8;
  uint64_t cnt[H] = {}, snap[H] = {};
#pragma unroll
  for (int j = 0; j < J; ++j) {
    if (j < n_groups) {  // the same for the whole workgroup
      const uint32_t first = uint32_t(j / R) * kChunkSlots + uint32_t(j % R) * kWave;
      const uint32_t bound = pad32 > first ? pad32 - first : 0u;  // lane_base < bound: before pad32
      const bool counted = lane_base < bound && idv[j] < n_experts;
      const uint32_t sh = (idv[j] & 7u) * 8u;
#pragma unroll
      for (int h = 0; h < H; ++h) {
        const bool in_h = H == 1 ? counted : (counted && (idv[j] >> 3) == uint32_t(h));
        cnt[h] += uint64_t(in_h ? 1u : 0u) << sh;
      }
      if (j + 1 == g_own) {
#pragma unroll
        for (int h = 0; h < H; ++h) snap[h] = cnt[h];
      }
    }
  }
  // wave sums: even and odd bytes widened to 16-bit fields (a field's sum is
  // at most 64 * 32), four 32-bit words per 8 experts: word 2p + (e >> 2)
  // holds expert e of parity p in its half (e >> 1) & 1
  {
    uint32_t packed[2][4 * H];
#pragma unroll
    for (int h = 0; h < H; ++h) {
#pragma unroll
      for (int which = 0; which < 2; ++which) {
        const uint64_t v = which ? snap[h] : cnt[h];
        const uint64_t ev = v & 0x00FF00FF00FF00FFull, od = (v >> 8) & 0x00FF00FF00FF00FFull;
        packed[which][4 * h + 0] = uint32_t(ev);
        packed[which][4 * h + 1] = uint32_t(ev >> 32);
        packed[which][4 * h + 2] = uint32_t(od);
        packed[which][4 * h + 3] = uint32_t(od >> 32);
      }
    }
#pragma unroll
    for (int which = 0; which < 2; ++which)
#pragma unroll
      for (int q = 0; q < 4 * H; ++q) {
        const uint32_t t = wave_inclusive_sum(packed[which][q]);
        if (lane == kWave - 1) wcount[which][wave][q] = t;
      }
  }
  __syncthreads();
  // expert b's count from a wave's packed words
  auto field = [](const uint32_t* words, int b) {
    const int e = b & 7;
    return (words[4 * (b >> 3) + 2 * (e & 1) + (e >> 2)] >> (16 * ((e >> 1) & 1))) & 0xFFFFu;
  };
  // wave 0: lane b < E sums expert b over the waves; the unrouted bucket
  // (lane E) is what the wave-wide sums of the routed counts leave
  if (wave == 0) {
    uint32_t t = 0, p = 0;
    if (lane < int(n_experts)) {
#pragma unroll
      for (int w = 0; w < kIdxWaves; ++w) {
        t += field(wcount[0][w], lane);
        p += field(wcount[1][w], lane);
      }
    }
    const uint32_t rt = __builtin_amdgcn_readlane(wave_inclusive_sum(t), kWave - 1);
    const uint32_t rp = __builtin_amdgcn_readlane(wave_inclusive_sum(p), kWave - 1);
    if (lane == int(n_experts)) {
      t = n32 - rt;
      p = uint32_t(c) * kChunkSlots - rp;
    }
    if (lane < nb) {  // nb <= 17
      tot[lane] = t;
      off[lane] = p;
    }
    // the chunk's starts and, in chunk 0, the CSR outputs, by this wave alone
    // while the other waves go on to their keys
    finalize_counts<kWave, 1>(tot, n_experts, base, esi, expert_ids, stats, soff, align, c == 0, off);
  }
  WaveTile<R> tile;
  wave_keys(own, wmap, n_slots, begin, n_experts, tile, pad_from);
  wave_count_keys(n_experts, nbits, whist, tile);
  __syncthreads();
  wave_scatter<false, R, kIdxThreads>(tile, n_experts, off, whist, teo, restore, n_slots);
}

// Rounds per chunk: up to kIdxChunk slots one workgroup takes them all; up to
// kIdxSmallMaxSlots, chunks of kIdxSmallRounds rounds put more workgroups on
// the few chunks there are; larger inputs use kIdxRounds.
int index_rounds(int64_t n_slots) {
  return (n_slots > kIdxChunk && n_slots <= kIdxSmallMaxSlots) ? kIdxSmallRounds : kIdxRounds;
}

int64_t index_chunks(int64_t n_slots) {
  const int64_t chunk = int64_t(kIdxThreads) * index_rounds(n_slots);
  return n_slots <= kIdxChunk ? 1 : (n_slots + chunk - 1) / chunk;
}

bool index_sum_path(int64_t n_slots, int n_experts) {
  const int64_t chunks = index_chunks(n_slots);
  const int64_t row = (int64_t(n_experts) + 8) & ~int64_t(7);  // E+1 rounded up to a multiple of 8
  return chunks > 1 && chunks <= kIdxSumMaxChunks && chunks * row <= kIdxSumMaxEntries;
}

// The few-expert pass takes chunks of kIdxSmallRounds rounds only (every
// input with so few chunks has them unless the build changes the limits), up
// to kIdxFewMaxGroups groups per wave at 8 experts or fewer and half that at
// 9 to 16, whose count costs twice as much per slot.
bool index_few_path(int64_t n_slots, int n_experts) {
  const int64_t chunks = index_chunks(n_slots);
  const int64_t max_groups = n_experts <= 8 ? kIdxFewMaxGroups : kIdxFewMaxGroups / 2;
  return chunks > 1 && n_experts <= kIdxFewMaxExperts && index_rounds(n_slots) == kIdxSmallRounds &&
         chunks * kIdxSmallRounds <= max_groups;
}

// Only the lookback path needs words past the fixed part.  Every input
// smaller than one that takes the lookback path takes either that path with
// fewer chunks or no lookback at all, so a workspace sized for some n_slots
// also fits every smaller one.
size_t index_workspace_bytes(int64_t n_slots, int n_experts) {
  const int64_t chunks = index_chunks(n_slots);
  if (chunks == 1 || index_sum_path(n_slots, n_experts)) return kWsFlags;
  const size_t c = size_t(chunks), nb = size_t(n_experts) + 1;
  return kWsFlags + align256(c * nb * 8);
}

IndexWorkspace index_workspace_carve(void* ws, int64_t n_slots, int n_experts) {
  (void)n_slots;
  (void)n_experts;
  char* p = static_cast<char*>(ws);
  IndexWorkspace w;
  w.err = reinterpret_cast<uint32_t*>(p);
  w.ticket = reinterpret_cast<uint32_t*>(p + 4);
  w.base = reinterpret_cast<uint32_t*>(p + kWsBase);
  w.counts = reinterpret_cast<uint16_t*>(p + kWsCounts);
  w.flags = reinterpret_cast<uint64_t*>(p + kWsFlags);
  return w;
}

// The two launches of the many-chunk path, chunks of R rounds.
template <typename IdT, int R>
hipError_t launch_chunks(const IdT* ids, int64_t n_slots, int n_experts, int nbits, int64_t chunks,
                         IndexWorkspace ws, uint32_t* esi, int32_t* expert_ids, uint32_t* stats,
                         uint32_t* soff, uint32_t align, uint32_t* teo, uint32_t* restore,
                         PadMask pad, IdT* wmap, hipStream_t s) {
  const int nb = n_experts + 1;
  hipLaunchKernelGGL((k_index_hist<IdT, R>), dim3(uint32_t(chunks)), dim3(kIdxThreads),
                     size_t(nb) * sizeof(uint32_t), s, ids, n_slots, uint32_t(n_experts), nbits,
                     chunks, ws, esi, expert_ids, stats, soff, align, pad, wmap);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_index_scatter<IdT, R>), dim3(uint32_t(chunks)), dim3(kIdxThreads),
                     size_t(1 + kIdxWaves) * nb * sizeof(uint32_t), s, ids, n_slots,
                     uint32_t(n_experts), nbits, ws, teo, restore);
  return hipGetLastError();
}

// The two launches of the wait-free path, chunks of R rounds.
template <typename IdT, int R>
hipError_t launch_sums(const IdT* ids, int64_t n_slots, int n_experts, int nbits, int64_t chunks,
                       IndexWorkspace ws, uint32_t* esi, int32_t* expert_ids, uint32_t* stats,
                       uint32_t* soff, uint32_t align, uint32_t* teo, uint32_t* restore,
                       PadMask pad, IdT* wmap, hipStream_t s) {
  const int nb = n_experts + 1, nbp = (nb + 7) & ~7;
  hipLaunchKernelGGL((k_index_count<IdT, R>), dim3(uint32_t(chunks)), dim3(kIdxThreads),
                     size_t(nb) * sizeof(uint32_t), s, ids, n_slots, uint32_t(n_experts), ws.counts,
                     pad, wmap);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t lds = size_t(2 * nbp + nb + kIdxWaves * nb) * sizeof(uint32_t);
  hipLaunchKernelGGL((k_index_scatter_sum<IdT, R>), dim3(uint32_t(chunks)), dim3(kIdxThreads), lds, s,
                     ids, n_slots, uint32_t(n_experts), nbits, int(chunks),
                     reinterpret_cast<const u32x4*>(ws.counts), esi, expert_ids, stats, soff, align,
                     teo, restore);
  return hipGetLastError();
}

// The one-launch pass for few experts, chunks of R rounds: NB counted
// buckets (8 or 16) and J groups per wave (8, 16 or 32; 8 or 16 at NB = 16),
// the fewest that hold the experts and the chunk rounds.
template <typename IdT, int R, int NB, int J>
hipError_t launch_few(const IdT* ids, int64_t n_slots, int n_experts, int nbits, int64_t chunks,
                      uint32_t* esi, int32_t* expert_ids, uint32_t* stats, uint32_t* soff,
                      uint32_t align, uint32_t* teo, uint32_t* restore, PadMask pad, IdT* wmap,
                      hipStream_t s) {
  const size_t lds = size_t(3 + kIdxWaves) * size_t(n_experts + 1) * sizeof(uint32_t);
  hipLaunchKernelGGL((k_index_few<IdT, R, NB, J>), dim3(uint32_t(chunks)), dim3(kIdxThreads), lds, s,
                     ids, n_slots, uint32_t(n_experts), nbits, int(chunks), esi, expert_ids, stats,
                     soff, align, teo, restore, pad, wmap);
  return hipGetLastError();
}

template <typename IdT, int R>
hipError_t launch_few_groups(const IdT* ids, int64_t n_slots, int n_experts, int nbits,
                             int64_t chunks, uint32_t* esi, int32_t* expert_ids, uint32_t* stats,
                             uint32_t* soff, uint32_t align, uint32_t* teo, uint32_t* restore,
                             PadMask pad, IdT* wmap, hipStream_t s) {
  const int64_t groups = chunks * R;
#define MOE_INDEX_FEW(NB, J) \
  launch_few<IdT, R, NB, J>(ids, n_slots, n_experts, nbits, chunks, esi, expert_ids, stats, soff, \
                            align, teo, restore, pad, wmap, s)
  if (n_experts <= 8) {
    if (groups <= 8) return MOE_INDEX_FEW(8, 8);
    if (groups <= 16) return MOE_INDEX_FEW(8, 16);
    return MOE_INDEX_FEW(8, 32);
  }
  if (groups <= 8) return MOE_INDEX_FEW(16, 8);
  return MOE_INDEX_FEW(16, 16);  // at most kIdxFewMaxGroups / 2 <= 16 groups
#undef MOE_INDEX_FEW
}

// The one-workgroup pass with T lanes.
template <typename IdT, int T>
hipError_t launch_one(const IdT* ids, int64_t n_slots, int n_experts, int nbits, uint32_t* esi,
                      int32_t* expert_ids, uint32_t* stats, uint32_t* soff, uint32_t align,
                      uint32_t* teo, uint32_t* restore, PadMask pad, IdT* wmap, hipStream_t s) {
  const size_t lds = size_t(2 + T / kWave) * size_t(n_experts + 1) * sizeof(uint32_t);
  hipLaunchKernelGGL((k_index_one<IdT, kIdxRounds, T>), dim3(1), dim3(T), lds, s, ids, n_slots,
                     uint32_t(n_experts), nbits, esi, expert_ids, stats, soff, align, teo, restore,
                     pad, wmap);
  return hipGetLastError();
}

template <typename IdT>
hipError_t launch_create_indices(const IdT* ids, int64_t n_slots, int n_experts, uint32_t* teo,
                                 uint32_t* esi, uint32_t* restore, int32_t* expert_ids,
                                 uint32_t* stats, uint32_t* soff, uint32_t align, void* wsp,
                                 PadMask pad, hipStream_t s) {
  const int64_t chunks = index_chunks(n_slots);
  const int nbits = 32 - __builtin_clz(uint32_t(n_experts));
  const IndexWorkspace ws = index_workspace_carve(wsp, n_slots, n_experts);
  // when masking, the map was handed in writable (the fused mask + index call)
  IdT* wmap = pad.count != nullptr ? const_cast<IdT*>(ids) : nullptr;
  if (chunks == 1) {
    // the fewest whole waves of kIdxRounds rounds that hold the slots
    const int64_t lanes = (n_slots + kIdxRounds - 1) / kIdxRounds;
#define MOE_INDEX_ONE(TT) \
  launch_one<IdT, TT>(ids, n_slots, n_experts, nbits, esi, expert_ids, stats, soff, align, teo, \
                      restore, pad, wmap, s)
    if (lanes <= 64) return MOE_INDEX_ONE(64);
    if (lanes <= 128) return MOE_INDEX_ONE(128);
    if (lanes <= 256) return MOE_INDEX_ONE(256);
    if (lanes <= 512) return MOE_INDEX_ONE(512);
    return MOE_INDEX_ONE(kIdxThreads);
#undef MOE_INDEX_ONE
  }
  if (index_few_path(n_slots, n_experts))
    return launch_few_groups<IdT, kIdxSmallRounds>(ids, n_slots, n_experts, nbits, chunks, esi,
                                                   expert_ids, stats, soff, align, teo, restore,
                                                   pad, wmap, s);
  if (index_sum_path(n_slots, n_experts)) {
    if (index_rounds(n_slots) == kIdxSmallRounds)
      return launch_sums<IdT, kIdxSmallRounds>(ids, n_slots, n_experts, nbits, chunks, ws, esi,
                                               expert_ids, stats, soff, align, teo, restore, pad,
                                               wmap, s);
    return launch_sums<IdT, kIdxRounds>(ids, n_slots, n_experts, nbits, chunks, ws, esi, expert_ids,
                                        stats, soff, align, teo, restore, pad, wmap, s);
  }
  if (index_rounds(n_slots) == kIdxSmallRounds)
    return launch_chunks<IdT, kIdxSmallRounds>(ids, n_slots, n_experts, nbits, chunks, ws, esi,
                                               expert_ids, stats, soff, align, teo, restore, pad,
                                               wmap, s);
  return launch_chunks<IdT, kIdxRounds>(ids, n_slots, n_experts, nbits, chunks, ws, esi, expert_ids,
                                        stats, soff, align, teo, restore, pad, wmap, s);
}

template hipError_t launch_create_indices<int32_t>(const int32_t*, int64_t, int, uint32_t*,
                                                   uint32_t*, uint32_t*, int32_t*, uint32_t*,
                                                   uint32_t*, uint32_t, void*, PadMask, hipStream_t);
template hipError_t launch_create_indices<int64_t>(const int64_t*, int64_t, int, uint32_t*,
                                                   uint32_t*, uint32_t*, int32_t*, uint32_t*,
                                                   uint32_t*, uint32_t, void*, PadMask, hipStream_t);

}  // namespace moe
