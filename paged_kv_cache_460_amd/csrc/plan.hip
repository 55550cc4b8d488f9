// Step planner: classify each sequence of the mixed step and lay out the work lists.
//
// A step mixes decode rows (one new token) with chunks of long prompts (restatement
// section 一, scheduler; section 二, item 1). All of it is planned on the device from
// the length arrays, so a step needs no host round trip:
//  * chunk sequences (two or more rows) are cut into tiles of prefill_rows_per_tile(G)
//    rows; tile_offsets[i] is the exclusive prefix sum of tiles, which lets the prefill
//    kernel map a flat task index to (sequence, tile);
//  * decode sequences (one row) are cut into KV partitions of P tokens. dec_tasks lists
//    every (sequence, partition) longest first: all full partitions, then the partial
//    last partitions in 32 length buckets, longest bucket first. Workgroups are
//    dispatched in list order, so the last ones to start are the shortest and the tail
//    of the decode launch is short. (The order inside a bucket depends on timing; each
//    task's result does not.)
//
// One workgroup of 1024 threads: each thread takes a contiguous run of sequences,
// counts, and after block-wide scans writes its entries.
#include "pa_internal.h"

namespace pa {

namespace {
constexpr int kBuckets = 32;

__device__ inline int block_exclusive_scan(int32_t* sums, int tid, int value, int& total) {
  sums[tid] = value;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int add = tid >= off ? sums[tid - off] : 0;
    __syncthreads();
    sums[tid] += add;
    __syncthreads();
  }
  total = sums[1023];
  const int excl = sums[tid] - value;
  __syncthreads();
  return excl;
}
}  // namespace

__global__ __launch_bounds__(1024) void plan_kernel(const int32_t* __restrict__ qsl,
                                                    const int32_t* __restrict__ seq_lens, int32_t num_seqs,
                                                    int32_t rows_per_tile, int32_t part_tokens, int32_t max_parts,
                                                    int32_t* __restrict__ tile_offsets,
                                                    int32_t* __restrict__ dec_tasks,
                                                    int32_t* __restrict__ dec_count) {
  __shared__ int32_t sums[1024];
  __shared__ int32_t bcount[kBuckets];
  __shared__ int32_t bfill[kBuckets];
  __shared__ int32_t boff[kBuckets];
  const int tid = threadIdx.x;
  if (tid < kBuckets) {
    bcount[tid] = 0;
    bfill[tid] = 0;
  }
  __syncthreads();
  const int per = (num_seqs + 1023) / 1024;
  const int b = tid * per;
  const int e = min(num_seqs, b + per);
  const int P = part_tokens;
  auto bucket_of = [&](int rem) { return (rem - 1) * kBuckets / P; };  // rem in [1, P)

  int tiles = 0, full = 0;
  for (int i = b; i < e; ++i) {
    const int n = qsl[i + 1] - qsl[i];
    if (n >= 2) {
      tiles += (n + rows_per_tile - 1) / rows_per_tile;
    } else if (n == 1) {
      const int L = seq_lens[i];
      full += L / P;
      if (L % P) atomicAdd(&bcount[bucket_of(L % P)], 1);
    }
  }
  int total_tiles, total_full;
  int tile_run = block_exclusive_scan(sums, tid, tiles, total_tiles);
  int full_run = block_exclusive_scan(sums, tid, full, total_full);
  if (tid == 0) {
    int run = total_full;
    for (int k = kBuckets - 1; k >= 0; --k) {
      boff[k] = run;
      run += bcount[k];
    }
    *dec_count = run;
    tile_offsets[num_seqs] = total_tiles;
  }
  __syncthreads();

  for (int i = b; i < e; ++i) {
    tile_offsets[i] = tile_run;
    const int n = qsl[i + 1] - qsl[i];
    if (n >= 2) {
      tile_run += (n + rows_per_tile - 1) / rows_per_tile;
    } else if (n == 1) {
      const int L = seq_lens[i];
      const int nfull = L / P;
      for (int q = 0; q < nfull; ++q) dec_tasks[full_run + q] = i * max_parts + q;
      full_run += nfull;
      if (L % P) {
        const int k = bucket_of(L % P);
        dec_tasks[boff[k] + atomicAdd(&bfill[k], 1)] = i * max_parts + nfull;
      }
    }
  }
}

hipError_t launch_plan(const AttnParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, stream, p.qsl, p.seq_lens, p.num_seqs,
                     prefill_rows_per_tile(p.group), p.part_tokens, p.max_parts, p.tile_offsets, p.dec_tasks,
                     p.dec_count);
  return hipGetLastError();
}

}  // namespace pa
