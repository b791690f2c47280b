// Host-side launchers of the routing kernels.  Arguments are validated by the
// C entry points before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// ---- index stage geometry -------------------------------------------------
// One workgroup of kIdxThreads threads owns a chunk of kIdxChunk consecutive
// slots; each of its waves owns kIdxRounds*64 consecutive slots of the chunk.
#ifndef MOE_IDX_THREADS
#define MOE_IDX_THREADS 1024
#endif
#ifndef MOE_IDX_ROUNDS
#define MOE_IDX_ROUNDS 2
#endif
// Inputs of (kIdxChunk, kIdxSmallMaxSlots] slots use chunks of
// kIdxSmallRounds rounds instead, so that more workgroups share them.
#ifndef MOE_IDX_SMALL_ROUNDS
#define MOE_IDX_SMALL_ROUNDS 1
#endif
#ifndef MOE_IDX_SMALL_MAX_SLOTS
#define MOE_IDX_SMALL_MAX_SLOTS 65536
#endif
constexpr int kIdxThreads = MOE_IDX_THREADS;
constexpr int kIdxWaves = kIdxThreads / 64;
constexpr int kIdxRounds = MOE_IDX_ROUNDS;
constexpr int kIdxSmallRounds = MOE_IDX_SMALL_ROUNDS;
constexpr int64_t kIdxSmallMaxSlots = MOE_IDX_SMALL_MAX_SLOTS;
constexpr int64_t kIdxChunk = int64_t(kIdxThreads) * kIdxRounds;
#define MOE_MAX_BUCKETS 1025  // experts + the unrouted bucket
// Inputs of up to kIdxSumMaxChunks chunks whose count table (chunks rows of
// E+1 16-bit counts, rows padded to a multiple of 8) holds at most
// kIdxSumMaxEntries entries take the wait-free path: every scatter workgroup
// sums the count table itself.  Larger inputs chain the chunks by lookback.
#ifndef MOE_IDX_SUM_MAX_CHUNKS
#define MOE_IDX_SUM_MAX_CHUNKS 512
#endif
#ifndef MOE_IDX_SUM_MAX_ENTRIES
#define MOE_IDX_SUM_MAX_ENTRIES (1 << 17)
#endif
// Inputs of at most kIdxFewMaxExperts experts and 2 to kIdxFewMaxGroups
// chunk rounds (chunks x rounds per chunk) take one launch in which every
// chunk workgroup counts all the slots itself, one ballot per expert
// (k_index_few).  0 turns that path off.
#ifndef MOE_IDX_FEW_MAX_GROUPS
#define MOE_IDX_FEW_MAX_GROUPS 32
#endif
#ifndef MOE_IDX_FEW_MAX_EXPERTS
#define MOE_IDX_FEW_MAX_EXPERTS 16
#endif
constexpr int64_t kIdxFewMaxGroups = MOE_IDX_FEW_MAX_GROUPS;
constexpr int kIdxFewMaxExperts = MOE_IDX_FEW_MAX_EXPERTS;
constexpr int64_t kIdxSumMaxChunks = MOE_IDX_SUM_MAX_CHUNKS;
constexpr int64_t kIdxSumMaxEntries = MOE_IDX_SUM_MAX_ENTRIES;
// Invariants the index kernels rely on, so that a sweep build with other
// values fails to compile instead of producing wrong indices:
//  - whole waves, at most 1024 lanes;
//  - the count table's rows hold 16-bit counts, so a chunk has at most 65535
//    slots (both chunk sizes);
//  - the table sums give each 16-byte column of a row (up to 129 of them at
//    1025 buckets, rounded up to whole waves: 192 lanes) at least one slice
//    of lanes.
static_assert(kIdxThreads % 64 == 0 && kIdxThreads <= 1024, "index workgroups are whole waves, at most 1024 lanes");
static_assert(kIdxRounds >= 1 && kIdxSmallRounds >= 1, "at least one round per chunk");
static_assert(kIdxChunk <= 65535 && int64_t(kIdxThreads) * kIdxSmallRounds <= 65535,
              "16-bit per-chunk counts");
static_assert(kIdxThreads >= (((MOE_MAX_BUCKETS + 7) / 8 + 63) / 64) * 64,
              "one slice of lanes per count-table column at the largest expert count");
static_assert(kIdxFewMaxGroups >= 0 && kIdxFewMaxGroups <= 32 && kIdxFewMaxExperts >= 1 &&
                  kIdxFewMaxExperts <= 16,
              "the few-expert pass holds at most 32 groups of ids and 16 expert counts per wave");

// The caller zero-fills the workspace once.  The kernels keep it ready for
// the next call of any shape: the last ticket holder resets the ticket, and
// the scatter kernel zeroes every lookback word of the call after reading it.
struct IndexWorkspace {
  uint32_t* err;        // [1]  sticky: bit 0 a cross-workgroup wait gave up, bit 1 a
                        //      ticket past the last chunk (workspace not zero-filled)
  uint32_t* ticket;     // [1]  chunk ticket counter
  uint32_t* base;       // [E+1]         first position of bucket b
  uint16_t* counts;     // [chunks][E+1 rounded up to a multiple of 8] slots per chunk and bucket
                        //      (wait-free path; rewritten by every call that uses it)
  uint64_t* flags;      // [chunks][E+1] (status << 32 | count) lookback words
};

// Workspace layout, the same for every shape: header words (error, ticket),
// bucket starts for the largest expert count, the count table at its
// largest, then the lookback words of the call.  The fixed part (up to the
// lookback words) is all that inputs taking the one-workgroup or the
// count-table path use, and they leave nothing in it that a later call reads.
constexpr size_t kWsHeader = 256;
constexpr size_t kWsBase = kWsHeader;
constexpr size_t kWsCounts = kWsBase + ((size_t(MOE_MAX_BUCKETS) * 4 + 255) & ~size_t(255));
constexpr size_t kWsFlags = kWsCounts + ((size_t(kIdxSumMaxEntries) * 2 + 255) & ~size_t(255));
constexpr size_t kIndexWorkspaceFixedBytes = kWsFlags;

int index_rounds(int64_t n_slots);
int64_t index_chunks(int64_t n_slots);
bool index_sum_path(int64_t n_slots, int n_experts);
bool index_few_path(int64_t n_slots, int n_experts);
size_t index_workspace_bytes(int64_t n_slots, int n_experts);
IndexWorkspace index_workspace_carve(void* ws, int64_t n_slots, int n_experts);

template <typename IdT>
hipError_t launch_mask_padding(IdT* ids, int64_t n_rows, int top_k, const int32_t* count,
                               int tp_rank, hipStream_t s);

// Padding rows masked while indexing (the fused mask + index call): rows r
// with r + tp_rank * (n_slots / top_k) >= *count become -1 in the map and
// are unrouted.  count == nullptr masks nothing and the map is only read.
struct PadMask {
  const int32_t* count;
  int32_t top_k;
  int32_t tp_rank;
};

template <typename IdT>
hipError_t launch_create_indices(const IdT* ids, int64_t n_slots, int n_experts, uint32_t* teo,
                                 uint32_t* esi, uint32_t* restore, int32_t* expert_ids,
                                 uint32_t* stats, uint32_t* scales_offset, uint32_t scales_align,
                                 void* ws, PadMask pad, hipStream_t s);

hipError_t launch_dispatch_bf16(const uint16_t* x, int64_t n_rows, int hidden, int top_k,
                                const uint32_t* restore, uint16_t* out, int64_t out_rows,
                                hipStream_t s);

hipError_t launch_dispatch_mxfp4(const uint16_t* x, int64_t n_rows, int hidden, int top_k,
                                 const uint32_t* restore, uint8_t* q, uint8_t* scales,
                                 int64_t out_rows, bool even_scale, bool packed, hipStream_t s);

// scale / residual: the fused epilogue (epilogue = false keeps the plain sum).
hipError_t launch_combine(const uint16_t* y, int64_t y_rows, const float* w,
                          const uint32_t* restore, int64_t n_rows, int hidden, int top_k,
                          bool epilogue, float scale, const uint16_t* residual, uint16_t* out,
                          hipStream_t s);

}  // namespace moe
