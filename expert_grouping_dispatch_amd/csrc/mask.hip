// Stage 1: padding rows of the routing map become -1
// ("core.transformer.moe.inference_routing_mask_kernel", mask_routing_padding).
#include "common.h"
#include "internal.h"

namespace moe {

// The boundary is computed on the device from the count behind the pointer,
// so a captured graph masks the right rows on every replay.  Threads stride
// over the entries from the first padding row on; earlier rows are
// never touched.
template <typename IdT>
__global__ __launch_bounds__(256) void k_mask_padding(IdT* __restrict__ ids, int64_t n_rows,
                                                      int top_k, const int32_t* __restrict__ count,
                                                      int tp_rank) {
  int64_t first = int64_t(*count) - int64_t(tp_rank) * n_rows;
  first = first < 0 ? 0 : (first > n_rows ? n_rows : first);
  const int64_t end = n_rows * top_k;
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t i = first * top_k + int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < end; i += stride)
    ids[i] = IdT(-1);
}

template <typename IdT>
hipError_t launch_mask_padding(IdT* ids, int64_t n_rows, int top_k, const int32_t* count,
                               int tp_rank, hipStream_t s) {
  const int64_t total = n_rows * top_k;
  if (total == 0) return hipSuccess;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  hipLaunchKernelGGL(k_mask_padding<IdT>, dim3(uint32_t(blocks)), dim3(256), 0, s, ids, n_rows,
                     top_k, count, tp_rank);
  return hipGetLastError();
}

template hipError_t launch_mask_padding<int32_t>(int32_t*, int64_t, int, const int32_t*, int,
                                                 hipStream_t);
template hipError_t launch_mask_padding<int64_t>(int64_t*, int64_t, int, const int32_t*, int,
                                                 hipStream_t);

}  // namespace moe
