// Step planner: classify each sequence of the mixed step and enumerate prefill tiles.
//
// A step mixes decode rows (one new token) with chunks of long prompts (restatement
// section 一, scheduler; section 二, item 1). Decode sequences need no list: the decode
// grid covers (sequence, partition, kv head) and idle entries exit at once. Chunk
// sequences (two or more rows) are cut into tiles of prefill_rows_per_tile(G) rows; this
// kernel writes the exclusive prefix sum of tiles per sequence, so the prefill kernel
// can map a flat task index to (sequence, tile) with no host round trip.
//
// One workgroup of 1024 threads: each thread sums a contiguous run of sequences, then
// a block-wide scan combines the runs.
#include "pa_internal.h"

namespace pa {

__global__ __launch_bounds__(1024) void plan_kernel(const int32_t* __restrict__ qsl, int32_t num_seqs,
                                                    int32_t rows_per_tile, int32_t* __restrict__ tile_offsets) {
  __shared__ int32_t sums[1024];
  const int tid = threadIdx.x;
  const int per = (num_seqs + 1023) / 1024;
  const int b = tid * per;
  const int e = min(num_seqs, b + per);
  int local = 0;
  for (int i = b; i < e; ++i) {
    const int n = qsl[i + 1] - qsl[i];
    local += (n >= 2) ? (n + rows_per_tile - 1) / rows_per_tile : 0;
  }
  sums[tid] = local;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int add = tid >= off ? sums[tid - off] : 0;
    __syncthreads();
    sums[tid] += add;
    __syncthreads();
  }
  int run = sums[tid] - local;
  for (int i = b; i < e; ++i) {
    tile_offsets[i] = run;
    const int n = qsl[i + 1] - qsl[i];
    run += (n >= 2) ? (n + rows_per_tile - 1) / rows_per_tile : 0;
  }
  if (tid == 1023) tile_offsets[num_seqs] = sums[1023];
}

hipError_t launch_plan(const AttnParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, stream, p.qsl, p.num_seqs,
                     prefill_rows_per_tile(p.group), p.tile_offsets);
  return hipGetLastError();
}

}  // namespace pa
