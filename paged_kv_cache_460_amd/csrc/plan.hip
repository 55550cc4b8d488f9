// Step planner: classify each sequence of the mixed step and lay out the work lists.
//
// A step mixes decode rows (one new token) with chunks of long prompts (restatement
// section 一, scheduler; section 二, item 1), and requests may list the same cached
// blocks for a shared prompt prefix (shengyayun.com blog, 关键实现细节 item 2). All of
// it is planned on the device from the length arrays and block tables, so a step needs
// no host round trip:
//  * chunk sequences (more than 16/G rows) are cut into tiles of prefill_rows_per_tile(G)
//    rows; tile_offsets[i] is the exclusive prefix sum of tiles, which lets the prefill
//    kernel map a flat task index to (sequence, tile);
//  * decode sequences (one row) are listed in dec_seqs. If all of them (two or more)
//    start with the same physical blocks, and those blocks hold only cached tokens of
//    every one of them, the common run of blocks is a shared prefix: it is attended
//    once for all decode rows together (the prefill kernel's prefix mode) and each
//    decode sequence keeps only its own suffix;
//  * sequences of 2..16/G rows (speculative verification) take the decode path as well:
//    their (row, head) pairs fill the MFMA columns and their whole KV range is cut
//    into partitions like a decode suffix;
//  * each decode suffix is cut into ceil(len / P) KV partitions of about equal length
//    (split_parts: whole 32-key steps, at most P). dec_tasks lists every (sequence,
//    partition) longest first: those of exactly P keys in sequence order, then the others
//    in 32 length buckets, longest bucket first. Workgroups are dispatched in list
//    order, so the last ones to start are the shortest and the tail of the decode launch
//    is short. (The order inside a bucket depends on timing; each task's result does
//    not.)
//
// One workgroup of 1024 threads: each thread takes a contiguous run of sequences,
// counts, and after block-wide scans and reductions writes its entries. A recorded step
// runs the planner in the same launch as the slot mapping and the cache write (the step
// prologue at the end of this file).
#include "cache_write.h"

namespace pa {

namespace {
constexpr int kBuckets = 32;
constexpr int kMinPrefixBlocks = 4;  // shorter shared runs are left to the decode kernel

// Block-wide exclusive scan and minimum for the 1024-thread planner: within each wave by
// cross-lane shuffles, then over the 16 wave results through LDS (two barriers each).
__device__ inline int block_exclusive_scan(int32_t* wsum, int tid, int value, int& total) {
  const int lane = tid & 63, w = tid >> 6;
  int v = value;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(v, off);
    if (lane >= off) v += t;
  }
  if (lane == 63) wsum[w] = v;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int x = wsum[k];
    before += k < w ? x : 0;
    all += x;
  }
  __syncthreads();  // wsum may be reused by the next call
  total = all;
  return before + v - value;
}

// The same scan over 64-bit values (partial-slot offsets).
__device__ inline int64_t block_exclusive_scan64(int64_t* wsum, int tid, int64_t value, int64_t& total) {
  const int lane = tid & 63, w = tid >> 6;
  int64_t v = value;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int64_t t = __shfl_up(v, off);
    if (lane >= off) v += t;
  }
  if (lane == 63) wsum[w] = v;
  __syncthreads();
  int64_t before = 0, all = 0;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int64_t x = wsum[k];
    before += k < w ? x : 0;
    all += x;
  }
  __syncthreads();
  total = all;
  return before + v - value;
}

__device__ inline int block_min(int32_t* wsum, int tid, int value) {
  const int lane = tid & 63, w = tid >> 6;
  int v = value;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = min(v, __shfl_xor(v, off));
  if (lane == 0) wsum[w] = v;
  __syncthreads();
  int r = wsum[0];
#pragma unroll
  for (int k = 1; k < 16; ++k) r = min(r, wsum[k]);
  __syncthreads();
  return r;
}
}  // namespace

// The planner, run by one workgroup of 1024 threads.
__device__ void plan_block(const AttnParams& p, int32_t rows_per_tile) {
  __shared__ int32_t sums[16];  // per-wave partial results of the block reductions
  __shared__ int64_t sums64[16];
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

  // A sequence of 2..16/G rows is a short multi-row step (speculative verification):
  // the decode kernel takes it, its (row, head) pairs filling the MFMA columns.
  const int G = p.group;
  auto is_multi = [&](int n) { return n >= 2 && n * G <= 16; };
  auto is_chunk = [&](int n) { return n >= 2 && n * G > 16; };

  // ---- prefill tiles, decode sequence list ----
  int tiles = 0, ndec = 0;
  for (int i = b; i < e; ++i) {
    const int n = qsl[i + 1] - qsl[i];
    if (is_chunk(n)) tiles += (n + rows_per_tile - 1) / rows_per_tile;
    else if (n == 1) ++ndec;
  }
  int total_tiles, total_dec;
  int tile_run = block_exclusive_scan(sums, tid, tiles, total_tiles);
  int dec_run = block_exclusive_scan(sums, tid, ndec, total_dec);
  for (int i = b; i < e; ++i) {
    p.tile_offsets[i] = tile_run;
    const int n = qsl[i + 1] - qsl[i];
    if (is_chunk(n)) tile_run += (n + rows_per_tile - 1) / rows_per_tile;
    else if (n == 1) p.dec_seqs[dec_run++] = i;
  }
  if (tid == 0) p.tile_offsets[num_seqs] = total_tiles;

  // ---- shared prefix: common leading blocks of every decode sequence ----
  // The first decode sequence is the reference (found by a block-wide min). Cheap test
  // first: every decode sequence must hold a cached block 0 equal to the reference's;
  // only then are all (sequence, block) pairs up to the shortest cached run compared,
  // in parallel, for the first mismatch.
  int my_first = 1 << 30;
  for (int i = b; i < e; ++i)
    if (qsl[i + 1] - qsl[i] == 1) {
      my_first = i;
      break;
    }
  const int ref = block_min(sums, tid, my_first);
  int prefix_blocks = 0;
  if (total_dec >= 2) {
    const int32_t* __restrict__ bref = p.block_tables + (int64_t)ref * MB;
    int cap_local = 1 << 30, same_first = 1;
    for (int i = b; i < e; ++i) {
      if (qsl[i + 1] - qsl[i] != 1) continue;
      const int cap = (seq_lens[i] - 1) / kBlock;  // blocks holding only cached tokens
      cap_local = min(cap_local, cap);
      if (cap == 0 || p.block_tables[(int64_t)i * MB] != bref[0]) same_first = 0;
    }
    const int cap = block_min(sums, tid, cap_local);
    const int all_same_first = block_min(sums, tid, same_first);
    if (all_same_first && cap >= kMinPrefixBlocks) {
      // Wave w compares sequences w, w + 16, ... four at a time, its lanes over the
      // blocks; each lane keeps the first mismatching block it saw. The comparisons are
      // selects, not branches, so all loads of a round are in flight together.
      const int lane = tid & 63, w = tid >> 6;
      int bad = cap;
      for (int i0 = w; i0 < num_seqs; i0 += 4 * 16) {
        bool dec[4];
        const int32_t* __restrict__ row[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = i0 + 16 * u;
          dec[u] = i < num_seqs && qsl[i + 1] - qsl[i] == 1;
          row[u] = p.block_tables + (int64_t)min(i, num_seqs - 1) * MB;
        }
        for (int c = lane; c < cap; c += 64) {
          const int r = bref[c];
          int x[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) x[u] = row[u][c];
#pragma unroll
          for (int u = 0; u < 4; ++u) bad = (dec[u] && x[u] != r) ? min(bad, c) : bad;
        }
      }
      prefix_blocks = block_min(sums, tid, bad);
    }
  }
  if (prefix_blocks < kMinPrefixBlocks) prefix_blocks = 0;
  int prefix_keys = prefix_blocks * kBlock;
  // Shared-prefix partitions: at least prefix_part_min keys each (a multiple of 64), and
  // at most max(kPrefixSlotRows / decode rows, 1) of them, which bounds the partials.
  int pparts = 0, pplen = 0;
  if (prefix_keys > 0) {
    const int pmin = p.prefix_part_min;
    int n = (prefix_keys + pmin - 1) / pmin;
    n = min(n, max(1, kPrefixSlotRows / total_dec));
    pplen = ((prefix_keys + n - 1) / n + 63) / 64 * 64;
    pparts = (prefix_keys + pplen - 1) / pplen;
  }

  // ---- decode-path tasks: partitions of each decode suffix [prefix_keys, L) and of each
  // multi-row sequence's whole range [0, L) ----
  auto task_len = [&](int i) {
    const int n = qsl[i + 1] - qsl[i];
    return n == 1 ? seq_lens[i] - prefix_keys : (is_multi(n) ? seq_lens[i] : 0);
  };
  // Partial slots of sequence i: nparts * Hkv * live columns when its result is split
  // over two or more partitions (shared-prefix ones included), else none.
  const int hkv = p.num_kv_heads;
  auto part_slots = [&](int i) -> int64_t {
    const int n = qsl[i + 1] - qsl[i];
    if (n != 1 && !is_multi(n)) return 0;
    const int nparts = (n == 1 ? pparts : 0) + split_parts(task_len(i), P).n;
    return nparts >= 2 ? (int64_t)nparts * hkv * n * G : 0;
  };
  // Tasks of exactly P keys come first, in sequence order; the others follow in 32 length
  // buckets, longest bucket first.
  auto bucket = [&](int tlen) { return (tlen - 1) * kBuckets / P; };
  auto tlen_of = [&](const PartSplit& sp, int len, int q) { return q + 1 < sp.n ? sp.plen : len - (sp.n - 1) * sp.plen; };
  int full = 0;
  int64_t my_slots = 0;
  for (int i = b; i < e; ++i) {
    const int len = task_len(i);
    const PartSplit sp = split_parts(len, P);
    for (int q = 0; q < sp.n; ++q) {
      const int t = tlen_of(sp, len, q);
      if (t == P) ++full;
      else atomicAdd(&bcount[bucket(t)], 1);
    }
    my_slots += part_slots(i);
  }
  int total_full;
  int full_run = block_exclusive_scan(sums, tid, full, total_full);
  int64_t total_slots;
  int64_t slot_run = block_exclusive_scan64(sums64, tid, my_slots, total_slots);
  // The host sizes the partial area from an upper bound over every plan of these sizes,
  // so this cannot overflow; if it ever did, nothing on the decode path runs (its rows
  // stay unwritten) rather than writing past the workspace.
  const bool overflow = total_slots > p.part_capacity;
  if (tid == 0) {
    int run = total_full;
    for (int k = kBuckets - 1; k >= 0; --k) {
      boff[k] = run;
      run += bcount[k];
    }
    p.plan_hdr[kHdrDecTasks] = overflow ? 0 : run;
    p.plan_hdr[kHdrDecSeqs] = total_dec;
    p.plan_hdr[kHdrPrefixKeys] = overflow ? 0 : prefix_keys;
    p.plan_hdr[kHdrPrefixParts] = overflow ? 0 : pparts;
    p.plan_hdr[kHdrPartSlots] = overflow ? -1 : (int)min(total_slots, (int64_t)INT32_MAX);
    p.plan_hdr[kHdrPrefixPartTokens] = pplen;
  }
  __syncthreads();
  for (int i = b; i < e; ++i) {
    const int len = task_len(i);
    const PartSplit sp = split_parts(len, P);
    for (int q = 0; q < sp.n; ++q) {
      const int t = tlen_of(sp, len, q);
      const int slot = t == P ? full_run++ : boff[bucket(t)] + atomicAdd(&bfill[bucket(t)], 1);
      p.dec_tasks[2 * slot] = i;
      p.dec_tasks[2 * slot + 1] = q;
    }
    p.part_base[i] = slot_run;
    slot_run += part_slots(i);
  }
}

__global__ __launch_bounds__(1024) void plan_kernel(AttnParams p, int32_t rows_per_tile) {
  plan_block(p, rows_per_tile);
}

hipError_t launch_plan(const AttnParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, stream, p, prefill_rows_per_tile(p.group));
  return hipGetLastError();
}

// ---- step prologue ----------------------------------------------------------------
// Slot mapping, cache write and planner of one step in a single launch of 1024-thread
// workgroups. They are independent of each other (the planner reads only the length
// arrays and block tables; the cache write needs the slots of its own 16 tokens, which
// it derives itself), and the attention kernels after them need all three, so one launch
// replaces three back-to-back ones. Workgroup 0 plans (when a plan is asked for); every
// other workgroup takes four cache-write units, one per 256 threads, each first writing
// the positions and slots of its 16 tokens (kv head 0 only) and keeping them in LDS.
// The results are those of the three separate launches, bit for bit.
template <int kElemBytes>
__global__ __launch_bounds__(1024) void step_prologue_kernel(PrologueArgs a, AttnParams p, int32_t rows_per_tile,
                                                             int32_t plan_wgs) {
  if ((int)blockIdx.x < plan_wgs) {
    plan_block(p, rows_per_tile);
    return;
  }
  __shared__ int64_t unit_slots[4][kWriteGroup];
  const int quarter = threadIdx.x >> 8, lt = threadIdx.x & 255;
  const int64_t unit = (int64_t)(blockIdx.x - plan_wgs) * 4 + quarter;
  const int64_t units = (a.num_tokens + kWriteGroup - 1) / kWriteGroup * a.num_kv_heads;
  const bool live = unit < units;
  const int h = live ? (int)(unit % a.num_kv_heads) : 0;
  const int64_t t0 = live ? unit / a.num_kv_heads * kWriteGroup : 0;
  if (lt < kWriteGroup) {
    const int64_t t = t0 + lt;
    int64_t slot = -1;
    if (live && t < a.num_tokens) {
      int32_t pos;
      slot = token_slot(a.block_tables, a.qsl, a.ctx, a.num_seqs, a.max_blocks, t, pos);
      if (h == 0) {
        if (a.positions) a.positions[t] = pos;
        a.slots[t] = slot;
      }
    }
    unit_slots[quarter][lt] = slot;
  }
  __syncthreads();
  if (!live) return;
  write_unit<kElemBytes>(static_cast<const uint8_t*>(a.k), static_cast<const uint8_t*>(a.v),
                         static_cast<uint8_t*>(a.k_cache), static_cast<uint8_t*>(a.v_cache), t0, h, a.num_tokens,
                         a.num_kv_heads, a.head_dim, lt, 256, [&](int j) { return unit_slots[quarter][j]; });
}

hipError_t launch_step_prologue(const PrologueArgs& a, const AttnParams* plan, hipStream_t stream) {
  const int64_t units = (a.num_tokens + kWriteGroup - 1) / kWriteGroup * a.num_kv_heads;
  const int32_t plan_wgs = plan ? 1 : 0;
  const int64_t grid = plan_wgs + (units + 3) / 4;
  if (grid == 0) return hipSuccess;
  const AttnParams p = plan ? *plan : AttnParams{};
  const int32_t rows = plan ? prefill_rows_per_tile(plan->group) : 0;
  if (a.elem_bytes == 2) {
    hipLaunchKernelGGL(step_prologue_kernel<2>, dim3((unsigned)grid), dim3(1024), 0, stream, a, p, rows, plan_wgs);
  } else {
    hipLaunchKernelGGL(step_prologue_kernel<4>, dim3((unsigned)grid), dim3(1024), 0, stream, a, p, rows, plan_wgs);
  }
  return hipGetLastError();
}

}  // namespace pa
