// Positions and slot mapping of a step's tokens (the slot rule is stated in
// cache_write.h).
//
// One thread per token; the owning sequence is found by binary search over
// query_start_loc. Integer work only, so the result is exact.
#include "cache_write.h"

namespace pa {

__global__ __launch_bounds__(256) void slot_mapping_kernel(
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ qsl,
    const int32_t* __restrict__ ctx, int32_t num_seqs, int32_t max_blocks, int64_t num_tokens,
    int32_t* __restrict__ positions, int64_t* __restrict__ slots) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= num_tokens) return;
  int32_t pos;
  const int64_t slot = token_slot(block_tables, qsl, ctx, num_seqs, max_blocks, t, pos);
  if (positions) positions[t] = pos;
  slots[t] = slot;
}

hipError_t launch_slot_mapping(const int32_t* block_tables, const int32_t* qsl, const int32_t* ctx,
                               int32_t num_seqs, int32_t max_blocks, int64_t num_tokens,
                               int32_t* positions, int64_t* slots, hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const int threads = 256;
  const int64_t blocks = (num_tokens + threads - 1) / threads;
  hipLaunchKernelGGL(slot_mapping_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream,
                     block_tables, qsl, ctx, num_seqs, max_blocks, num_tokens, positions, slots);
  return hipGetLastError();
}

}  // namespace pa
