// Positions and slot mapping of a step's tokens.
//
// The worker builds, for every token of the step, its position and the cache slot its
// K/V go to before the forward pass (hn.213312.xyz restatement of "Inside vLLM",
// section 一, forward pass). Blocks hold 16 tokens (shengyayun.com blog, 关键实现细节
// item 1). Slot = block id * 16 + position within the block.
//
// One thread per token; the owning sequence is found by binary search over
// query_start_loc. Integer work only, so the result is exact.
#include "pa_internal.h"

namespace pa {

__global__ __launch_bounds__(256) void slot_mapping_kernel(
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ qsl,
    const int32_t* __restrict__ ctx, int32_t num_seqs, int32_t max_blocks, int64_t num_tokens,
    int32_t* __restrict__ positions, int64_t* __restrict__ slots) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= num_tokens) return;
  if (num_seqs == 0 || t >= qsl[num_seqs]) {
    if (positions) positions[t] = 0;
    slots[t] = -1;
    return;
  }
  const int i = upper_index(qsl, num_seqs, t);
  const int64_t pos = (int64_t)ctx[i] + (t - qsl[i]);
  const int64_t block = block_tables[(int64_t)i * max_blocks + pos / kBlock];
  if (positions) positions[t] = (int32_t)pos;
  slots[t] = block * kBlock + pos % kBlock;
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
