// Step planner: classify each sequence of the mixed step and lay out the work lists.
//
// A step mixes decode rows (one new token) with chunks of long prompts (restatement
// section 一, scheduler; section 二, item 1), and requests may list the same cached
// blocks for a shared prompt prefix (shengyayun.com blog, 关键实现细节 item 2). All of
// it is planned on the device from the length arrays and block tables, so a step needs
// no host round trip:
//  * chunk sequences (two or more rows) are cut into tiles of prefill_rows_per_tile(G)
//    rows; tile_offsets[i] is the exclusive prefix sum of tiles, which lets the prefill
//    kernel map a flat task index to (sequence, tile);
//  * decode sequences (one row) are listed in dec_seqs. If all of them (two or more)
//    start with the same physical blocks, and those blocks hold only cached tokens of
//    every one of them, the common run of blocks is a shared prefix: it is attended
//    once for all decode rows together (the prefill kernel's prefix mode) and each
//    decode sequence keeps only its own suffix;
//  * each decode suffix is cut into KV partitions of P tokens. dec_tasks lists every
//    (sequence, partition) longest first: all full partitions, then the partial last
//    partitions in 32 length buckets, longest bucket first. Workgroups are dispatched in
//    list order, so the last ones to start are the shortest and the tail of the decode
//    launch is short. (The order inside a bucket depends on timing; each task's result
//    does not.)
//
// One workgroup of 1024 threads: each thread takes a contiguous run of sequences,
// counts, and after block-wide scans and reductions writes its entries.
#include "pa_internal.h"

namespace pa {

namespace {
constexpr int kBuckets = 32;
constexpr int kMinPrefixBlocks = 4;  // shorter shared runs are left to the decode kernel

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

__device__ inline int block_min(int32_t* sums, int tid, int value) {
  sums[tid] = value;
  __syncthreads();
  for (int off = 512; off > 0; off >>= 1) {
    if (tid < off) sums[tid] = min(sums[tid], sums[tid + off]);
    __syncthreads();
  }
  const int r = sums[0];
  __syncthreads();
  return r;
}
}  // namespace

__global__ __launch_bounds__(1024) void plan_kernel(AttnParams p, int32_t rows_per_tile) {
  __shared__ int32_t sums[1024];
  __shared__ int32_t bcount[kBuckets];
  __shared__ int32_t bfill[kBuckets];
  __shared__ int32_t boff[kBuckets];
  const int32_t* __restrict__ qsl = p.qsl;
  const int32_t* __restrict__ seq_lens = p.seq_lens;
  const int num_seqs = p.num_seqs;
  const int tid = threadIdx.x;
  if (tid < kBuckets) {
    bcount[tid] = 0;
    bfill[tid] = 0;
  }
  const int per = (num_seqs + 1023) / 1024;
  const int b = tid * per;
  const int e = min(num_seqs, b + per);
  const int P = p.part_tokens;
  const int MB = p.max_blocks;

  // ---- prefill tiles, decode sequence list ----
  int tiles = 0, ndec = 0;
  for (int i = b; i < e; ++i) {
    const int n = qsl[i + 1] - qsl[i];
    if (n >= 2) tiles += (n + rows_per_tile - 1) / rows_per_tile;
    else if (n == 1) ++ndec;
  }
  int total_tiles, total_dec;
  int tile_run = block_exclusive_scan(sums, tid, tiles, total_tiles);
  int dec_run = block_exclusive_scan(sums, tid, ndec, total_dec);
  for (int i = b; i < e; ++i) {
    p.tile_offsets[i] = tile_run;
    const int n = qsl[i + 1] - qsl[i];
    if (n >= 2) tile_run += (n + rows_per_tile - 1) / rows_per_tile;
    else if (n == 1) p.dec_seqs[dec_run++] = i;
  }
  if (tid == 0) p.tile_offsets[num_seqs] = total_tiles;

  // ---- shared prefix: common leading blocks of every decode sequence ----
  // The first decode sequence is the reference (found by a block-wide min, not read
  // back from dec_seqs).
  int my_first = 1 << 30;
  for (int i = b; i < e; ++i)
    if (qsl[i + 1] - qsl[i] == 1) {
      my_first = i;
      break;
    }
  const int ref = block_min(sums, tid, my_first);
  int lcp = 1 << 30;
  if (total_dec >= 2) {
    const int32_t* __restrict__ bref = p.block_tables + (int64_t)ref * MB;
    for (int i = b; i < e; ++i) {
      if (qsl[i + 1] - qsl[i] != 1) continue;
      const int cap = (seq_lens[i] - 1) / kBlock;  // blocks holding only cached tokens
      const int32_t* __restrict__ bi = p.block_tables + (int64_t)i * MB;
      int c = 0;
      while (c < cap && bi[c] == bref[c]) ++c;
      lcp = min(lcp, c);
    }
  }
  int prefix_blocks = total_dec >= 2 ? block_min(sums, tid, lcp) : 0;
  if (prefix_blocks < kMinPrefixBlocks) prefix_blocks = 0;
  const int prefix_keys = prefix_blocks * kBlock;

  // ---- decode tasks over each suffix [prefix_keys, L) ----
  int full = 0;
  for (int i = b; i < e; ++i) {
    if (qsl[i + 1] - qsl[i] != 1) continue;
    const int len = seq_lens[i] - prefix_keys;
    full += len / P;
    if (len % P) atomicAdd(&bcount[(len % P - 1) * kBuckets / P], 1);
  }
  int total_full;
  int full_run = block_exclusive_scan(sums, tid, full, total_full);
  if (tid == 0) {
    int run = total_full;
    for (int k = kBuckets - 1; k >= 0; --k) {
      boff[k] = run;
      run += bcount[k];
    }
    p.plan_hdr[kHdrDecTasks] = run;
    p.plan_hdr[kHdrDecSeqs] = total_dec;
    p.plan_hdr[kHdrPrefixKeys] = prefix_keys;
    p.plan_hdr[kHdrPrefixParts] = (prefix_keys + P - 1) / P;
  }
  __syncthreads();
  for (int i = b; i < e; ++i) {
    if (qsl[i + 1] - qsl[i] != 1) continue;
    const int len = seq_lens[i] - prefix_keys;
    const int nfull = len / P;
    for (int q = 0; q < nfull; ++q) p.dec_tasks[full_run + q] = i * p.max_parts + q;
    full_run += nfull;
    if (len % P) {
      const int k = (len % P - 1) * kBuckets / P;
      p.dec_tasks[boff[k] + atomicAdd(&bfill[k], 1)] = i * p.max_parts + nfull;
    }
  }
}

hipError_t launch_plan(const AttnParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, stream, p, prefill_rows_per_tile(p.group));
  return hipGetLastError();
}

}  // namespace pa
