// C entry points: argument checks, the gfx950 device check, then the launch.
// Nothing here allocates, synchronises or reads device memory.
#include <atomic>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "internal.h"
#include "moe_route.h"

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_device_ok[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// The kernels are written for gfx950 only; any other device is rejected
// rather than run on code built for another target.  For tests of this
// rejection, MOE_ROUTE_ASSUME_ARCH (when set) stands in for the device's
// architecture name.
int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return MOE_ERR_UNSUPPORTED_DEVICE;
  int state = dev < kMaxDevices ? g_device_ok[dev].load(std::memory_order_relaxed) : 0;
  if (state == 0) {
    hipDeviceProp_t prop;
    state = 2;
    if (hipGetDeviceProperties(&prop, dev) == hipSuccess) {
      const char* forced = std::getenv("MOE_ROUTE_ASSUME_ARCH");
      const char* a = forced != nullptr ? forced : prop.gcnArchName;
      if (std::strncmp(a, "gfx950", 6) == 0 && (a[6] == '\0' || a[6] == ':')) state = 1;
    }
    if (dev < kMaxDevices) g_device_ok[dev].store(state, std::memory_order_relaxed);
  }
  return state == 1 ? MOE_OK : MOE_ERR_UNSUPPORTED_DEVICE;
}

int launched(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH; }

bool slots_ok(int64_t n_rows, int32_t top_k) {
  if (n_rows < 0 || top_k < 1 || top_k > MOE_MAX_TOP_K) return false;
  return n_rows <= int64_t(0xFFFFFFFEu) / top_k;  // every slot index and position < sentinel
}

template <typename IdT>
int mask_padding(IdT* routing_map, int64_t n_rows, int32_t top_k, const int32_t* real_token_count,
                 int32_t tp_rank, void* stream) {
  if (!slots_ok(n_rows, top_k) || tp_rank < 0 || real_token_count == nullptr ||
      !aligned(real_token_count, 4))
    return MOE_ERR_INVALID_ARGUMENT;
  if (n_rows > 0 && (routing_map == nullptr || !aligned(routing_map, sizeof(IdT))))
    return MOE_ERR_INVALID_ARGUMENT;
  if (const int d = check_device()) return d;
  return launched(moe::launch_mask_padding(routing_map, n_rows, top_k, real_token_count, tp_rank,
                                           static_cast<hipStream_t>(stream)));
}

// The argument checks of the index entry points, workspace aside.
template <typename IdT>
int index_arguments(const IdT* topk_ids, int64_t n_slots, int32_t n_experts,
                    const uint32_t* token_expert_order, const uint32_t* expert_start_indices,
                    const uint32_t* restore_token_order, const int32_t* expert_ids,
                    const uint32_t* expert_usage_stats, const uint32_t* scales_offset,
                    uint32_t scales_align) {
  if (n_slots < 0 || n_slots > int64_t(0xFFFFFFFEu) || n_experts < 1 || n_experts > MOE_MAX_EXPERTS)
    return MOE_ERR_INVALID_ARGUMENT;
  if (expert_start_indices == nullptr || expert_ids == nullptr || expert_usage_stats == nullptr)
    return MOE_ERR_INVALID_ARGUMENT;
  if (n_slots > 0 && (topk_ids == nullptr || token_expert_order == nullptr ||
                      restore_token_order == nullptr))
    return MOE_ERR_INVALID_ARGUMENT;
  if (scales_offset != nullptr &&
      (scales_align < 1 || uint64_t(n_slots) + uint64_t(n_experts) * scales_align >= 0xFFFFFFFFull))
    return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(topk_ids, sizeof(IdT)) || !aligned(token_expert_order, 4) ||
      !aligned(expert_start_indices, 4) || !aligned(restore_token_order, 4) ||
      !aligned(expert_ids, 4) || !aligned(expert_usage_stats, 4) || !aligned(scales_offset, 4))
    return MOE_ERR_INVALID_ARGUMENT;
  return MOE_OK;
}

template <typename IdT>
int create_indices(const IdT* topk_ids, int64_t n_slots, int32_t n_experts,
                   uint32_t* token_expert_order, uint32_t* expert_start_indices,
                   uint32_t* restore_token_order, int32_t* expert_ids,
                   uint32_t* expert_usage_stats, uint32_t* scales_offset, uint32_t scales_align,
                   void* workspace, size_t workspace_bytes, moe::PadMask pad, void* stream) {
  if (const int a = index_arguments(topk_ids, n_slots, n_experts, token_expert_order, expert_start_indices,
                                    restore_token_order, expert_ids, expert_usage_stats, scales_offset,
                                    scales_align))
    return a;
  if (workspace == nullptr || !aligned(workspace, 256)) return MOE_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < moe::index_workspace_bytes(n_slots, n_experts))
    return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (const int d = check_device()) return d;
  return launched(moe::launch_create_indices(topk_ids, n_slots, n_experts, token_expert_order,
                                             expert_start_indices, restore_token_order, expert_ids,
                                             expert_usage_stats, scales_offset, scales_align,
                                             workspace, pad, static_cast<hipStream_t>(stream)));
}

// Stages 1 and 2 in one call: the mask's checks, then the index checks on
// the n_rows * top_k slots of the map.
template <typename IdT>
int mask_create_indices(IdT* routing_map, int64_t n_rows, int32_t top_k,
                        const int32_t* real_token_count, int32_t tp_rank, int32_t n_experts,
                        uint32_t* token_expert_order, uint32_t* expert_start_indices,
                        uint32_t* restore_token_order, int32_t* expert_ids,
                        uint32_t* expert_usage_stats, uint32_t* scales_offset,
                        uint32_t scales_align, void* workspace, size_t workspace_bytes,
                        void* stream) {
  if (!slots_ok(n_rows, top_k) || tp_rank < 0 || real_token_count == nullptr ||
      !aligned(real_token_count, 4))
    return MOE_ERR_INVALID_ARGUMENT;
  return create_indices<IdT>(routing_map, n_rows * top_k, n_experts, token_expert_order,
                             expert_start_indices, restore_token_order, expert_ids,
                             expert_usage_stats, scales_offset, scales_align, workspace,
                             workspace_bytes, moe::PadMask{real_token_count, top_k, tp_rank},
                             stream);
}

// ---- scratch of moe_create_indices_noalloc --------------------------------
// For callers that cannot allocate, the index stage's scratch is this
// file-scope device array instead of a caller's workspace: one copy per GPU,
// held from the library's load until the process ends.  Its size is the
// fixed part of the index workspace, which is all that inputs taking the
// one-workgroup, the few-expert (none of it) or the count-table path use;
// those paths rewrite everything they read from it within the call, so
// nothing in it needs clearing between calls.  In host code the array's name stands for a host-side shadow:
// kernels get only the device address looked up below.
constexpr size_t kScratchBytes = moe::kIndexWorkspaceFixedBytes;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
std::atomic<void*> g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device

// The device address of `scratch` on device `dev` (the current device), looked
// up on the first call on that device and kept; nullptr if the lookup fails.
void* scratch_address(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  return p;
}

int combine(const uint16_t* y, int64_t y_rows, const float* router_weights,
            const uint32_t* restore_token_order, int64_t n_rows, int32_t hidden, int32_t top_k,
            bool epilogue, float scale, const uint16_t* residual, uint16_t* output_tokens,
            void* stream) {
  if (!slots_ok(n_rows, top_k) || hidden <= 0 || hidden % 8 != 0 || y_rows < 0)
    return MOE_ERR_INVALID_ARGUMENT;
  if (n_rows > 0 && (router_weights == nullptr || restore_token_order == nullptr ||
                     output_tokens == nullptr))
    return MOE_ERR_INVALID_ARGUMENT;
  if (y_rows > 0 && y == nullptr) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(y, 16) || !aligned(output_tokens, 16) || !aligned(router_weights, 4) ||
      !aligned(restore_token_order, 4) || !aligned(residual, 16))
    return MOE_ERR_INVALID_ARGUMENT;
  if (residual != nullptr && n_rows > 0) {  // the residual rows must not overlap the output
    const uintptr_t bytes = uintptr_t(n_rows) * uintptr_t(hidden) * 2;
    const uintptr_t r = reinterpret_cast<uintptr_t>(residual), o = reinterpret_cast<uintptr_t>(output_tokens);
    if (r < o + bytes && o < r + bytes) return MOE_ERR_INVALID_ARGUMENT;
  }
  if (const int d = check_device()) return d;
  return launched(moe::launch_combine(y, y_rows, router_weights, restore_token_order, n_rows,
                                      hidden, top_k, epilogue, scale, residual, output_tokens,
                                      static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

const char* moe_error_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARGUMENT: return "invalid argument";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MOE_ERR_UNSUPPORTED_DEVICE: return "unsupported device (gfx950 required)";
    case MOE_ERR_LAUNCH: return "kernel launch failed";
    case MOE_ERR_SCRATCH_LIMIT:
      return "input too large for the static scratch of moe_create_indices_noalloc (needs the lookback path)";
    default: return "unknown status";
  }
}

int moe_mask_padding(int32_t* routing_map, int64_t n_rows, int32_t top_k,
                     const int32_t* real_token_count, int32_t tp_rank, void* stream) {
  return mask_padding(routing_map, n_rows, top_k, real_token_count, tp_rank, stream);
}

int moe_mask_padding_i64(int64_t* routing_map, int64_t n_rows, int32_t top_k,
                         const int32_t* real_token_count, int32_t tp_rank, void* stream) {
  return mask_padding(routing_map, n_rows, top_k, real_token_count, tp_rank, stream);
}

size_t moe_create_indices_workspace_bytes(int64_t n_slots, int32_t n_experts) {
  if (n_slots < 0 || n_slots > int64_t(0xFFFFFFFEu) || n_experts < 1 || n_experts > MOE_MAX_EXPERTS)
    return 0;
  return moe::index_workspace_bytes(n_slots, n_experts);
}

int moe_create_indices(const int32_t* topk_ids, int64_t n_slots, int32_t n_experts,
                       uint32_t* token_expert_order, uint32_t* expert_start_indices,
                       uint32_t* restore_token_order, int32_t* expert_ids,
                       uint32_t* expert_usage_stats, uint32_t* scales_offset,
                       uint32_t scales_align, void* workspace, size_t workspace_bytes,
                       void* stream) {
  return create_indices(topk_ids, n_slots, n_experts, token_expert_order, expert_start_indices,
                        restore_token_order, expert_ids, expert_usage_stats, scales_offset,
                        scales_align, workspace, workspace_bytes, moe::PadMask{nullptr, 1, 0},
                        stream);
}

int moe_create_indices_noalloc(const int32_t* topk_ids, int64_t n_slots, int32_t n_experts,
                               uint32_t* token_expert_order, uint32_t* expert_start_indices,
                               uint32_t* restore_token_order, int32_t* expert_ids,
                               uint32_t* expert_usage_stats, uint32_t* scales_offset,
                               uint32_t scales_align, void* stream) {
  if (const int a = index_arguments(topk_ids, n_slots, n_experts, token_expert_order, expert_start_indices,
                                    restore_token_order, expert_ids, expert_usage_stats, scales_offset,
                                    scales_align))
    return a;
  if (moe::index_workspace_bytes(n_slots, n_experts) > kScratchBytes) return MOE_ERR_SCRATCH_LIMIT;
  if (const int d = check_device()) return d;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_LAUNCH;
  void* ws = scratch_address(dev);
  if (ws == nullptr) return MOE_ERR_LAUNCH;
  return launched(moe::launch_create_indices(topk_ids, n_slots, n_experts, token_expert_order,
                                             expert_start_indices, restore_token_order, expert_ids,
                                             expert_usage_stats, scales_offset, scales_align, ws,
                                             moe::PadMask{nullptr, 1, 0}, static_cast<hipStream_t>(stream)));
}

int moe_create_indices_i64(const int64_t* topk_ids, int64_t n_slots, int32_t n_experts,
                           uint32_t* token_expert_order, uint32_t* expert_start_indices,
                           uint32_t* restore_token_order, int32_t* expert_ids,
                           uint32_t* expert_usage_stats, uint32_t* scales_offset,
                           uint32_t scales_align, void* workspace, size_t workspace_bytes,
                           void* stream) {
  return create_indices(topk_ids, n_slots, n_experts, token_expert_order, expert_start_indices,
                        restore_token_order, expert_ids, expert_usage_stats, scales_offset,
                        scales_align, workspace, workspace_bytes, moe::PadMask{nullptr, 1, 0},
                        stream);
}

int moe_mask_create_indices(int32_t* routing_map, int64_t n_rows, int32_t top_k,
                            const int32_t* real_token_count, int32_t tp_rank, int32_t n_experts,
                            uint32_t* token_expert_order, uint32_t* expert_start_indices,
                            uint32_t* restore_token_order, int32_t* expert_ids,
                            uint32_t* expert_usage_stats, uint32_t* scales_offset,
                            uint32_t scales_align, void* workspace, size_t workspace_bytes,
                            void* stream) {
  return mask_create_indices(routing_map, n_rows, top_k, real_token_count, tp_rank, n_experts,
                             token_expert_order, expert_start_indices, restore_token_order,
                             expert_ids, expert_usage_stats, scales_offset, scales_align,
                             workspace, workspace_bytes, stream);
}

int moe_mask_create_indices_i64(int64_t* routing_map, int64_t n_rows, int32_t top_k,
                                const int32_t* real_token_count, int32_t tp_rank,
                                int32_t n_experts, uint32_t* token_expert_order,
                                uint32_t* expert_start_indices, uint32_t* restore_token_order,
                                int32_t* expert_ids, uint32_t* expert_usage_stats,
                                uint32_t* scales_offset, uint32_t scales_align, void* workspace,
                                size_t workspace_bytes, void* stream) {
  return mask_create_indices(routing_map, n_rows, top_k, real_token_count, tp_rank, n_experts,
                             token_expert_order, expert_start_indices, restore_token_order,
                             expert_ids, expert_usage_stats, scales_offset, scales_align,
                             workspace, workspace_bytes, stream);
}

int moe_dispatch(const uint16_t* input_tokens, int64_t n_rows, int32_t hidden, int32_t top_k,
                 const uint32_t* restore_token_order, uint16_t* out, int64_t out_rows,
                 void* stream) {
  if (!slots_ok(n_rows, top_k) || hidden <= 0 || hidden % 8 != 0 || out_rows < 0)
    return MOE_ERR_INVALID_ARGUMENT;
  if (n_rows > 0 && (input_tokens == nullptr || restore_token_order == nullptr))
    return MOE_ERR_INVALID_ARGUMENT;
  if (out_rows > 0 && out == nullptr) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(input_tokens, 16) || !aligned(out, 16) || !aligned(restore_token_order, 4))
    return MOE_ERR_INVALID_ARGUMENT;
  if (const int d = check_device()) return d;
  return launched(moe::launch_dispatch_bf16(input_tokens, n_rows, hidden, top_k,
                                            restore_token_order, out, out_rows,
                                            static_cast<hipStream_t>(stream)));
}

int moe_dispatch_mxfp4(const uint16_t* input_tokens, int64_t n_rows, int32_t hidden,
                       int32_t top_k, const uint32_t* restore_token_order, uint8_t* out_q,
                       uint8_t* out_scales, int64_t out_rows, uint32_t flags, void* stream) {
  const bool packed = (flags & MOE_MXFP4_PACKED_ROWS) != 0;
  if (!slots_ok(n_rows, top_k) || hidden <= 0 || hidden % MOE_MXFP4_BLOCK != 0 || out_rows < 0 ||
      (flags & ~(MOE_MXFP4_EVEN_SCALE | MOE_MXFP4_PACKED_ROWS)) != 0)
    return MOE_ERR_INVALID_ARGUMENT;
  if (packed && (hidden % 512 != 0 || out_scales != nullptr)) return MOE_ERR_INVALID_ARGUMENT;
  if (n_rows > 0 && (input_tokens == nullptr || restore_token_order == nullptr))
    return MOE_ERR_INVALID_ARGUMENT;
  if (out_rows > 0 && (out_q == nullptr || (!packed && out_scales == nullptr)))
    return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(input_tokens, 16) || !aligned(out_q, 16) || !aligned(restore_token_order, 4))
    return MOE_ERR_INVALID_ARGUMENT;
  if (const int d = check_device()) return d;
  return launched(moe::launch_dispatch_mxfp4(input_tokens, n_rows, hidden, top_k,
                                             restore_token_order, out_q, out_scales, out_rows,
                                             (flags & MOE_MXFP4_EVEN_SCALE) != 0, packed,
                                             static_cast<hipStream_t>(stream)));
}

int moe_combine(const uint16_t* y, int64_t y_rows, const float* router_weights,
                const uint32_t* restore_token_order, int64_t n_rows, int32_t hidden,
                int32_t top_k, uint16_t* output_tokens, void* stream) {
  return combine(y, y_rows, router_weights, restore_token_order, n_rows, hidden, top_k, false,
                 1.0f, nullptr, output_tokens, stream);
}

int moe_combine_epilogue(const uint16_t* y, int64_t y_rows, const float* router_weights,
                         const uint32_t* restore_token_order, int64_t n_rows, int32_t hidden,
                         int32_t top_k, float scale, const uint16_t* residual,
                         uint16_t* output_tokens, void* stream) {
  return combine(y, y_rows, router_weights, restore_token_order, n_rows, hidden, top_k, true,
                 scale, residual, output_tokens, stream);
}

}  // extern "C"
