/*
 * moe_route.h -- C ABI of the MI355X (gfx950) MoE token-routing library.
 *
 * One GPU's share of the Mixture-of-Experts routing path, in four stages:
 *   1. moe_mask_padding     -- padding rows of the routing map become -1
 *   2. moe_create_indices   -- expert-grouped (stable) slot order, CSR starts,
 *                              inverse map, active-expert list, usage stats
 *   3. moe_dispatch         -- token rows copied into an expert-contiguous
 *      moe_dispatch_mxfp4      buffer, as bf16 or as MXFP4
 *   4. moe_combine          -- weighted sum of expert outputs back per token
 * plus moe_mask_create_indices, stages 1 and 2 in one call, and
 * moe_create_indices_noalloc, stage 2 for callers that cannot allocate.
 *
 * Conventions shared by every entry point
 *   - Pointers marked [device] are device (HBM) pointers on the current HIP
 *     device; [host] pointers are ordinary host memory.  The caller allocates
 *     and owns every buffer; the library never allocates, never frees and
 *     keeps no pointer after a call returns.
 *   - Tensors are dense and row-major.  bf16 values are passed as their
 *     16-bit patterns (uint16_t).
 *   - `stream` is a hipStream_t of the current device (NULL = the legacy
 *     default stream); the device check looks at the current device.  Work
 *     is enqueued asynchronously; no call synchronises with the host or
 *     reads device data on the host, so a whole sequence can be captured
 *     into a HIP graph.
 *   - Calls keep no state between them outside the buffers passed, so calls
 *     on different streams may run at once, except that calls sharing an
 *     index workspace must not overlap, and neither may calls of
 *     moe_create_indices_noalloc on one GPU (they share its static scratch).
 *   - A slot is the pair (token t, choice j) with flat index i = t*top_k + j.
 *     MOE_SENTINEL (0xFFFFFFFF) marks "no slot / no position".
 *   - Return value: MOE_OK, or an error code with nothing enqueued.  Errors
 *     are argument errors detected on the host (null or misaligned pointer,
 *     size out of range), an undersized workspace (or an input too large for
 *     the static scratch of moe_create_indices_noalloc), a device that is not
 *     gfx950 (rejected, never emulated), or a failed launch.  For tests of
 *     that rejection, the environment variable MOE_ROUTE_ASSUME_ARCH, when
 *     set, stands in for the device's architecture name (read once per
 *     device and process).  Bad *data*
 *     (an expert id outside [0, n_experts), a position outside the output
 *     buffer) is not an error: such a slot is treated as unrouted.
 */
#ifndef MOE_ROUTE_H
#define MOE_ROUTE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_SENTINEL 0xFFFFFFFFu
#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_TOP_K 1024
#define MOE_MXFP4_BLOCK 32

/* moe_dispatch_mxfp4 flags */
#define MOE_MXFP4_EVEN_SCALE 1u  /* "even-mode" scale exponent (see moe_dispatch_mxfp4) */
#define MOE_MXFP4_PACKED_ROWS 2u /* payload and scales packed into one row per slot */

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = 1,
  MOE_ERR_WORKSPACE_TOO_SMALL = 2,
  MOE_ERR_UNSUPPORTED_DEVICE = 3,
  MOE_ERR_LAUNCH = 4,
  MOE_ERR_SCRATCH_LIMIT = 5 /* input larger than moe_create_indices_noalloc's static scratch */
} moe_status;

/* Static, human-readable text for a status code. [host] */
const char* moe_error_string(int status);

/*
 * Stage 1 -- mask padding rows of the routing map, in place.
 * ("core.transformer.moe.inference_routing_mask_kernel", mask_routing_padding:
 *  rows of a CUDA-graph-padded routing map at or past the real token count
 *  get -1 in every top-k slot; the count is read on the device; local row r
 *  is global row r + tp_rank*n_rows.)
 *
 *   routing_map       [device] int32 [n_rows, top_k], modified in place.
 *   n_rows            N >= 0, rows of the (padded) local routing map.
 *   top_k             1 <= top_k <= MOE_MAX_TOP_K.
 *   real_token_count  [device] int32[1], the real token count in the global
 *                     frame.  Read by the kernel, so only the value behind
 *                     the pointer needs to change between graph replays.
 *                     Values beyond the rows of this shard mask nothing or
 *                     everything (the boundary is clamped to [0, N]).
 *   tp_rank           >= 0, this shard's index in its SP/TP group.
 * Rows before the boundary are neither read nor written.
 */
int moe_mask_padding(int32_t* routing_map, int64_t n_rows, int32_t top_k,
                     const int32_t* real_token_count, int32_t tp_rank, void* stream);

/*
 * As moe_mask_padding for an int64 routing map [n_rows, top_k] (the dtype of
 * the routing map on the mask page's mask_routing_padding parameters).
 */
int moe_mask_padding_i64(int64_t* routing_map, int64_t n_rows, int32_t top_k,
                         const int32_t* real_token_count, int32_t tp_rank, void* stream);

/*
 * Size in bytes of the scratch workspace moe_create_indices needs for
 * n_slots slots and n_experts experts (0 if the sizes are out of range). [host]
 */
size_t moe_create_indices_workspace_bytes(int64_t n_slots, int32_t n_experts);

/*
 * Stage 2 -- group routed slots by expert.
 * ("moe_create_indices", description and Args: histogram the expert ids,
 *  scan the histogram into CSR offsets, scatter; outputs token_expert_order,
 *  expert_start_indices, restore_token_order, expert_ids,
 *  expert_usage_stats.)
 *
 *   topk_ids              [device] int32 [n_slots] (the masked routing map
 *                         viewed flat, slot i = t*top_k + j).  A slot is
 *                         routed iff 0 <= id < n_experts.
 *   n_slots               S, 0 <= S <= 0xFFFFFFFE.
 *   n_experts             E, 1 <= E <= MOE_MAX_EXPERTS.
 *   token_expert_order    [device] uint32 [S] out: entries [0, V) are the
 *                         routed slot indices ordered by (expert id, slot
 *                         index) -- a stable grouping; entries [V, S) are
 *                         MOE_SENTINEL.  V = number of routed slots.
 *   expert_start_indices  [device] uint32 [E+1] out: CSR starts over the
 *                         active experts (those with >= 1 slot), in
 *                         ascending id order; entry A.. E hold V.
 *   restore_token_order   [device] uint32 [S] out: position of slot i in
 *                         token_expert_order, MOE_SENTINEL if unrouted.
 *   expert_ids            [device] int32 [E] out: active expert ids in
 *                         ascending order, then -1.
 *   expert_usage_stats    [device] uint32 [2] out: {largest number of slots
 *                         on one expert, number of active experts A}.
 *   scales_offset         [device] uint32 [E+1] out, or NULL ("moe_create_indices",
 *                         Args: scales_offset_p, the aligned scale offsets for
 *                         block-scaled grouped matmul): entry j < A is the sum over
 *                         active experts j' < j of their slot count rounded up
 *                         to a multiple of scales_align; entries A..E hold the
 *                         total.  Offsets are in rows; a block-scaled GEMM
 *                         multiplies by its bytes per scale row.
 *   scales_align          >= 1 when scales_offset is given (ignored otherwise);
 *                         S + E*scales_align must stay below 2^32.
 *   workspace             [device] scratch of at least
 *                         moe_create_indices_workspace_bytes(S, E) bytes,
 *                         256-byte aligned, zero-filled once before its first
 *                         use; every call leaves it ready for the next one
 *                         (its layout does not depend on S and E, and a call
 *                         reads nothing an earlier call left in it, so any S
 *                         and E that fit its size may follow).
 *                         Calls that share a workspace must not overlap.
 *                         Its first 32-bit word becomes nonzero (and stays
 *                         so) if a cross-workgroup wait ever gave up or the
 *                         call found the workspace not in the state a
 *                         zero-filled one is left in; the outputs of such a
 *                         call are unspecified, but every access stays
 *                         inside the buffers passed.
 * All outputs are fully written, also when S = 0 or V = 0.
 */
int moe_create_indices(const int32_t* topk_ids, int64_t n_slots, int32_t n_experts,
                       uint32_t* token_expert_order, uint32_t* expert_start_indices,
                       uint32_t* restore_token_order, int32_t* expert_ids,
                       uint32_t* expert_usage_stats, uint32_t* scales_offset,
                       uint32_t scales_align, void* workspace, size_t workspace_bytes,
                       void* stream);

/*
 * As moe_create_indices, with no workspace argument and no allocation of any
 * kind: for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation).  The
 * index stage's scratch is a static device array of the library, one per
 * GPU, of 266752 bytes (the fixed part of the workspace), held from the
 * library's load until the process ends.  Arguments, layouts, results and
 * the other errors are those of moe_create_indices.
 *
 * Limit: the input must take a path of the index stage that needs no
 * lookback words (the one-workgroup, few-expert or count-table path):
 * n_slots <= 2048, or at most 512 chunks (of 1024 slots up
 * to 65536 slots, of 2048 slots above) whose count table, with
 * n_experts + 1 rounded up to a multiple of 8 entries per chunk, holds at
 * most 131072 entries.  That is up to 1,015,808 slots at n_experts = 256,
 * 1,048,576 at n_experts <= 255 (for n_experts + 1 <= 256 entries), and
 * 260,096 at n_experts = 1024.  Larger inputs return MOE_ERR_SCRATCH_LIMIT
 * with nothing enqueued; moe_create_indices with a workspace takes them.
 * Those paths leave nothing in the scratch that a later call reads, so
 * nothing needs clearing between calls.
 *
 * All calls on one GPU share its scratch: calls that overlap in time on one
 * GPU (on different streams, or from different threads) race and give
 * unspecified results.  The first call on a GPU looks up the scratch's
 * device address (not a stream operation); if a runtime refuses that lookup
 * during stream capture, make one call outside capture first.
 */
int moe_create_indices_noalloc(const int32_t* topk_ids, int64_t n_slots, int32_t n_experts,
                               uint32_t* token_expert_order, uint32_t* expert_start_indices,
                               uint32_t* restore_token_order, int32_t* expert_ids,
                               uint32_t* expert_usage_stats, uint32_t* scales_offset,
                               uint32_t scales_align, void* stream);

/* As moe_create_indices for int64 expert ids (topk_ids [n_slots] int64). */
int moe_create_indices_i64(const int64_t* topk_ids, int64_t n_slots, int32_t n_experts,
                           uint32_t* token_expert_order, uint32_t* expert_start_indices,
                           uint32_t* restore_token_order, int32_t* expert_ids,
                           uint32_t* expert_usage_stats, uint32_t* scales_offset,
                           uint32_t scales_align, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * Stages 1 and 2 in one call, for callers that run them back to back.
 * ("core.transformer.moe.inference_routing_mask_kernel", mask_routing_padding,
 *  then "moe_create_indices", as above.)  The results are exactly those of
 * moe_mask_padding(routing_map, n_rows, top_k, real_token_count, tp_rank)
 * followed by moe_create_indices on the masked map viewed flat
 * (n_slots = n_rows * top_k), with one kernel launch fewer: padding slots
 * are set to -1 in routing_map (in place) and counted as unrouted while the
 * index is built.  Arguments, layouts, ownership and errors are those of the
 * two calls; the map must not be read or written by other work while the
 * call runs.
 */
int moe_mask_create_indices(int32_t* routing_map, int64_t n_rows, int32_t top_k,
                            const int32_t* real_token_count, int32_t tp_rank, int32_t n_experts,
                            uint32_t* token_expert_order, uint32_t* expert_start_indices,
                            uint32_t* restore_token_order, int32_t* expert_ids,
                            uint32_t* expert_usage_stats, uint32_t* scales_offset,
                            uint32_t scales_align, void* workspace, size_t workspace_bytes,
                            void* stream);

/* As moe_mask_create_indices for an int64 routing map. */
int moe_mask_create_indices_i64(int64_t* routing_map, int64_t n_rows, int32_t top_k,
                                const int32_t* real_token_count, int32_t tp_rank,
                                int32_t n_experts, uint32_t* token_expert_order,
                                uint32_t* expert_start_indices, uint32_t* restore_token_order,
                                int32_t* expert_ids, uint32_t* expert_usage_stats,
                                uint32_t* scales_offset, uint32_t scales_align, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * Stage 3a -- dispatch in bf16.
 * ("Struct_ep_dispatch_async_mxfp4", execute and Args: input_tokens
 *  [num_tokens, hidden_size] are sent to the experts chosen in topk_ids
 *  [num_tokens, top_k]; this is one GPU's local share, with the receive
 *  buffer laid out expert-contiguously.)
 *
 *   input_tokens          [device] bf16 [n_rows, hidden], 16-byte aligned.
 *   n_rows, hidden, top_k N >= 0; hidden > 0 and a multiple of 8;
 *                         1 <= top_k <= MOE_MAX_TOP_K.
 *   restore_token_order   [device] uint32 [n_rows*top_k] from
 *                         moe_create_indices.
 *   out                   [device] bf16 [out_rows, hidden], 16-byte aligned.
 *                         Row p = restore_token_order[t*top_k+j] receives
 *                         a bit copy of input row t.  Rows no slot points to
 *                         are left untouched; positions >= out_rows are
 *                         skipped.
 */
int moe_dispatch(const uint16_t* input_tokens, int64_t n_rows, int32_t hidden, int32_t top_k,
                 const uint32_t* restore_token_order, uint16_t* out, int64_t out_rows,
                 void* stream);

/*
 * Stage 3b -- dispatch in MXFP4.
 * ("Struct_ep_dispatch_async_mxfp4", execute: tokens are transferred as FP4
 *  quants with scales; Parameters dispatch_dtype / dispatch_scale_dtype.)
 * Each 32-element block of a row is encoded once and written to every
 * position the row's slots map to:
 *   scale exponent  se = clamp(floor(log2(max |x|)) - 2, -127, 127),
 *                   se = -127 for an all-zero block; stored as se + 127.
 *                   With MOE_MXFP4_EVEN_SCALE (the page names per-token
 *                   even-mode scales without defining them; read here as:
 *                   round max |x| to E2M1's one mantissa bit, halves up,
 *                   before the floor):
 *                   floor(log2(max |x|)) gains 1 when the mantissa fraction
 *                   of max |x| is >= 0.75, so a block maximum that would
 *                   scale into [7, 8) lands in [3.5, 4) instead.
 *   element code    nearest of {0, .5, 1, 1.5, 2, 3, 4, 6} to |x| * 2^-se,
 *                   ties to the even code, values above 6 saturate to 6;
 *                   bit 3 = sign bit of x (kept on zero).
 *   byte m of a block = code(2m) | code(2m+1) << 4.
 * Inputs must be finite.
 *
 *   input_tokens, n_rows, top_k, restore_token_order  as moe_dispatch.
 *   hidden        > 0, a multiple of 32 (of 512 with MOE_MXFP4_PACKED_ROWS).
 *   out_q         [device] uint8 [out_rows, hidden/2], 16-byte aligned; with
 *                 MOE_MXFP4_PACKED_ROWS uint8 [out_rows, hidden/2 + hidden/32]
 *                 holding each slot's payload followed by its scale bytes
 *                 (the page has the scales travel with the FP4 quants).
 *   out_scales    [device] uint8 [out_rows, hidden/32]; NULL with
 *                 MOE_MXFP4_PACKED_ROWS.
 *   flags         0, or an OR of MOE_MXFP4_EVEN_SCALE and MOE_MXFP4_PACKED_ROWS.
 */
int moe_dispatch_mxfp4(const uint16_t* input_tokens, int64_t n_rows, int32_t hidden,
                       int32_t top_k, const uint32_t* restore_token_order, uint8_t* out_q,
                       uint8_t* out_scales, int64_t out_rows, uint32_t flags, void* stream);

/*
 * Stage 4 -- combine.
 * ("Struct_ep_combine_wait", execute and Args: the weighted sum of the
 *  routed expert outputs of each token with its router weights
 *  [num_tokens, top_k], into output_tokens [num_tokens, hidden_size].)
 *
 *   out[t] = bf16( sum_{j = 0..top_k-1, slot routed} w[t,j] * y[restore[t*top_k+j]] )
 * in fp32, acc starting at +0, j ascending, every product and sum rounded
 * on its own (no fused multiply-add), bf16 round-to-nearest-even at the end.
 * Rows without a routed slot are written as +0.
 *
 *   y                     [device] bf16 [y_rows, hidden], expert outputs in
 *                         expert-grouped row order, 16-byte aligned.
 *   router_weights        [device] fp32 [n_rows, top_k].
 *   restore_token_order   [device] uint32 [n_rows*top_k]; positions
 *                         >= y_rows are skipped like unrouted slots.
 *   output_tokens         [device] bf16 [n_rows, hidden], 16-byte aligned.
 *   hidden                > 0, a multiple of 8.
 */
int moe_combine(const uint16_t* y, int64_t y_rows, const float* router_weights,
                const uint32_t* restore_token_order, int64_t n_rows, int32_t hidden,
                int32_t top_k, uint16_t* output_tokens, void* stream);

/*
 * Combine with an elementwise epilogue fused in ("Struct_ep_combine_wait",
 * Parameters: has_epilogue_fusion applies an elementwise function after the
 * weighted sum).  The epilogue here is a scale and an optional residual add:
 *   out[t] = bf16( fl(fl(scale * acc[t]) + residual[t]) )     (residual given)
 *   out[t] = bf16( fl(scale * acc[t]) )                       (residual NULL)
 * with acc[t] the fp32 sum of moe_combine, every operation rounded on its
 * own.  scale = 1 and residual = NULL give exactly moe_combine.
 *   residual      [device] bf16 [n_rows, hidden], 16-byte aligned, or NULL;
 *                 must not overlap output_tokens.
 * Other arguments as moe_combine.
 */
int moe_combine_epilogue(const uint16_t* y, int64_t y_rows, const float* router_weights,
                         const uint32_t* restore_token_order, int64_t n_rows, int32_t hidden,
                         int32_t top_k, float scale, const uint16_t* residual,
                         uint16_t* output_tokens, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_ROUTE_H */
