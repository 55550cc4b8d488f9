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
//    partition) as a DecTask record, longest first: those of exactly P keys in sequence
//    order, then the others in 32 length buckets, longest bucket first. Workgroups are
//    dispatched in list order, so the last ones to start are the shortest and the tail
//    of the decode launch is short. (The order inside a bucket depends on timing; each
//    task's result does not.)
//
// One workgroup of 1024 threads: each thread takes a contiguous run of sequences,
// counts, and after block-wide scans and reductions writes its entries. A recorded step
// runs the planner in the same launch as the slot mapping and the cache write (the step
// prologue at the end of this file).
#include "cache_write.h"

namespace pa {

namespace {
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
constexpr int kBuckets = 32;
constexpr int kMinPrefixBlocks = 4;  // shorter shared runs are left to the decode kernel
constexpr int kLdsSeqs = 2048;       // sequences whose lengths the planner stages in LDS

// Inclusive scans over the lanes of a wave by DPP lane shifts, which run on the VALU
// with no LDS traffic (cross-lane shuffles through LDS, issued by all 16 waves of the
// planner at once, kept its LDS pipe busy for microseconds per reduction): within each
// row of 16 lanes by shifts of 1, 2, 4 and 8, then across rows by broadcasting lane 15
// into rows 1 and 3 and lane 31 into rows 2 and 3. Lanes without a source add 0 (sum)
// or keep their own value (minimum).
__device__ inline int row_scan_add(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  return v;
}
__device__ inline int wave_scan_add(int v) {
  v = row_scan_add(v);
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2, 3
  return v;
}
__device__ inline int row_scan_min(int v) {
  v = min(v, __builtin_amdgcn_update_dpp(v, v, 0x111, 0xf, 0xf, false));
  v = min(v, __builtin_amdgcn_update_dpp(v, v, 0x112, 0xf, 0xf, false));
  v = min(v, __builtin_amdgcn_update_dpp(v, v, 0x114, 0xf, 0xf, false));
  v = min(v, __builtin_amdgcn_update_dpp(v, v, 0x118, 0xf, 0xf, false));
  return v;
}
__device__ inline int wave_scan_min(int v) {
  v = row_scan_min(v);
  v = min(v, __builtin_amdgcn_update_dpp(v, v, 0x142, 0xa, 0xf, false));
  v = min(v, __builtin_amdgcn_update_dpp(v, v, 0x143, 0xc, 0xf, false));
  return v;
}

// Workgroup barrier that orders LDS accesses only. The planner never reads back the
// global stores it makes, so its barriers need not wait for them to complete (a full
// __syncthreads would).
__device__ inline void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Block-wide reductions for the 1024-thread planner, several 32-bit values at a time:
// within each wave by DPP scans, then over the 16 wave results (one per lane of the first
// row, scanned once more); two LDS barriers per call, whatever the number of values.
// Exclusive scans (and totals) of the first NS values, minimums of the next NM.
template <int NS, int NM>
__device__ inline void block_scan_min(int32_t (*red)[8], int tid, const int32_t* sv, int32_t* before, int32_t* total,
                                      int32_t* mv) {
  static_assert(NS + NM <= 8, "at most 8 values per call");
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  int32_t inc[NS > 0 ? NS : 1];
#pragma unroll
  for (int k = 0; k < NS; ++k) inc[k] = wave_scan_add(sv[k]);
#pragma unroll
  for (int k = 0; k < NM; ++k) mv[k] = wave_scan_min(mv[k]);
  if (lane == 63) {
#pragma unroll
    for (int k = 0; k < NS; ++k) red[w][k] = inc[k];
#pragma unroll
    for (int k = 0; k < NM; ++k) red[w][NS + k] = mv[k];
  }
  lds_barrier();
#pragma unroll
  for (int k = 0; k < NS; ++k) {
    const int32_t x = row_scan_add(lane < 16 ? red[lane][k] : 0);  // inclusive over the waves
    total[k] = __builtin_amdgcn_readlane(x, 15);
    const int32_t bw = w > 0 ? __builtin_amdgcn_readlane(x, w - 1) : 0;
    before[k] = bw + inc[k] - sv[k];
  }
#pragma unroll
  for (int k = 0; k < NM; ++k) mv[k] = __builtin_amdgcn_readlane(row_scan_min(lane < 16 ? red[lane][NS + k] : INT32_MAX), 15);
  lds_barrier();  // red may be reused by the next call
}
}  // namespace

// The planner, run by one workgroup of 1024 threads.
__device__ void plan_block(const AttnParams& p, int32_t rows_per_tile) {
  __shared__ int32_t red[16][8];  // per-wave partial results of the block reductions
  __shared__ int32_t bcount[kBuckets];
  __shared__ int32_t bfill[kBuckets];
  __shared__ int32_t boff[kBuckets];
  // First query row, query rows, length and first block id of each sequence, staged
  // once (steps of up to kLdsSeqs sequences; larger ones read them from memory each time).
  __shared__ int32_t s_q0[kLdsSeqs], s_rows[kLdsSeqs], s_len[kLdsSeqs], s_b0[kLdsSeqs];
  const int32_t* __restrict__ qsl = p.qsl;
  const int32_t* __restrict__ seq_lens = p.seq_lens;
  const int num_seqs = p.num_seqs;
  const int tid = threadIdx.x;
  const int MB = p.max_blocks;
  const int hkv = p.num_kv_heads;
  const bool staged = num_seqs <= kLdsSeqs;
  if (tid < kBuckets) {
    bcount[tid] = 0;
    bfill[tid] = 0;
  }
  if (staged) {
    for (int i = tid; i < num_seqs; i += 1024) {
      s_q0[i] = qsl[i];
      s_rows[i] = qsl[i + 1] - qsl[i];
      s_len[i] = seq_lens[i];
      s_b0[i] = p.block_tables[(int64_t)i * MB];
    }
  }
  lds_barrier();
  auto q0_of = [&](int i) { return staged ? s_q0[i] : qsl[i]; };
  auto rows_of = [&](int i) { return staged ? s_rows[i] : qsl[i + 1] - qsl[i]; };
  auto len_of = [&](int i) { return staged ? s_len[i] : seq_lens[i]; };
  auto b0_of = [&](int i) { return staged ? s_b0[i] : p.block_tables[(int64_t)i * MB]; };
  const int per = (num_seqs + 1023) / 1024;
  const int b = tid * per;
  const int e = min(num_seqs, b + per);

  // A sequence of 2..16/G rows is a short multi-row step (speculative verification):
  // the decode kernel takes it, its (row, head) pairs filling the MFMA columns.
  const int G = p.group;
  auto is_multi = [&](int n) { return n >= 2 && n * G <= 16; };
  auto is_chunk = [&](int n) { return n >= 2 && n * G > 16; };

  // ---- one pass over the sequences: prefill tiles, decode rows, decode-path keys, and
  // what the shared-prefix test needs (first decode row, shortest cached run, range of
  // first block ids) ----
  // Keys are counted in whole 32-key steps (an upper bound on the keys), so that every
  // sum fits 32 bits.
  constexpr int32_t kBig = INT32_MAX;
  int32_t cnt[4] = {0, 0, 0, 0};  // tiles, decode rows, decode-row key steps, multi-row key steps
  int32_t mins[4] = {kBig, kBig, kBig, kBig};  // first decode row, cached blocks, min b0, -max b0
  for (int i = b; i < e; ++i) {
    const int n = rows_of(i);
    if (is_chunk(n)) {
      cnt[0] += (n + rows_per_tile - 1) / rows_per_tile;
    } else if (n == 1) {
      const int L = len_of(i), b0 = b0_of(i);
      cnt[1] += 1;
      cnt[2] += (L + 31) / 32;
      mins[0] = min(mins[0], i);
      mins[1] = min(mins[1], (L - 1) / kBlock);  // blocks holding only cached tokens
      mins[2] = min(mins[2], b0);
      mins[3] = min(mins[3], -b0);
    } else if (is_multi(n)) {
      cnt[3] += (len_of(i) + 31) / 32;
    }
  }
  int32_t before[4], total[4];
  block_scan_min<4, 4>(red, tid, cnt, before, total, mins);
  const int total_tiles = total[0], total_dec = total[1];
  {
    int tile_run = before[0], dec_run = before[1];
    for (int i = b; i < e; ++i) {
      p.tile_offsets[i] = tile_run;
      const int n = rows_of(i);
      if (is_chunk(n)) tile_run += (n + rows_per_tile - 1) / rows_per_tile;
      else if (n == 1) p.dec_seqs[dec_run++] = i;
    }
  }
  if (tid == 0) p.tile_offsets[num_seqs] = total_tiles;

  // ---- shared prefix: common leading blocks of every decode sequence ----
  // Cheap test first: every decode row holds at least kMinPrefixBlocks cached blocks and
  // all start with the same block; only then are all (sequence, block) pairs up to the
  // shortest cached run compared with the first decode row's, in parallel, for the first
  // mismatch.
  int prefix_blocks = 0;
  const int cap = mins[1];
  if (total_dec >= 2 && mins[2] == -mins[3] && cap >= kMinPrefixBlocks) {
    const int32_t* __restrict__ bref = p.block_tables + (int64_t)mins[0] * MB;
    // Each lane keeps the first mismatching block it saw. The comparisons are selects, not
    // branches, so all loads of a round are in flight together.
    const int lane = tid & 63, w = tid >> 6;
    int bad = cap;
    // Rows of 16-byte-aligned tables (aligned base, width a multiple of 4) are compared
    // four blocks per 16-byte load: wave w takes sequences w, w + 16, ... eight at a time,
    // lane l blocks c0 + 4l .. c0 + 4l + 3 of each (c0 + 4l < cap <= MB, and both are
    // multiples of 4, so all four lie in the row); blocks past the run are not counted.
    const bool vec = MB % 4 == 0 && (reinterpret_cast<uintptr_t>(p.block_tables) & 15) == 0;
    if (vec) {
      for (int i0 = w; i0 < num_seqs; i0 += 8 * 16) {
        bool dec[8];
        const int32_t* __restrict__ row[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int i = min(i0 + 16 * u, num_seqs - 1);
          dec[u] = i0 + 16 * u < num_seqs && rows_of(i) == 1;
          row[u] = p.block_tables + (int64_t)i * MB;
        }
        for (int c0 = 4 * lane; c0 < cap; c0 += 4 * 64) {
          const i32x4 r = *reinterpret_cast<const i32x4*>(bref + c0);
          i32x4 x[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) x[u] = *reinterpret_cast<const i32x4*>(row[u] + c0);
#pragma unroll
          for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int u = 0; u < 8; ++u)
              bad = (c0 + e < cap && dec[u] && x[u][e] != r[e]) ? min(bad, c0 + e) : bad;
        }
      }
    } else {
      // Otherwise four sequences at a time, each lane four blocks 64 apart per round.
      // (Indices past the run are clamped to its last block: every table row holds
      // MB >= cap entries.)
      for (int i0 = w; i0 < num_seqs; i0 += 4 * 16) {
        bool dec[4];
        const int32_t* __restrict__ row[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = min(i0 + 16 * u, num_seqs - 1);
          dec[u] = i0 + 16 * u < num_seqs && rows_of(i) == 1;
          row[u] = p.block_tables + (int64_t)i * MB;
        }
        for (int c0 = lane; c0 < cap; c0 += 4 * 64) {
          int r[4], x[4][4];
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int cc = min(c0 + 64 * v, cap - 1);
            r[v] = bref[cc];
#pragma unroll
            for (int u = 0; u < 4; ++u) x[u][v] = row[u][cc];
          }
#pragma unroll
          for (int v = 0; v < 4; ++v)
#pragma unroll
            for (int u = 0; u < 4; ++u) bad = (dec[u] && x[u][v] != r[v]) ? min(bad, c0 + 64 * v) : bad;
        }
      }
    }
    int32_t m[1] = {bad};
    block_scan_min<0, 1>(red, tid, nullptr, nullptr, nullptr, m);
    prefix_blocks = m[0];
  }
  if (prefix_blocks < kMinPrefixBlocks) prefix_blocks = 0;
  const int prefix_keys = prefix_blocks * kBlock;

  // ---- decode-path tasks: partitions of each decode suffix [prefix_keys, L) and of each
  // multi-row sequence's whole range [0, L) ----
  auto task_len = [&](int i) {
    const int n = rows_of(i);
    return n == 1 ? len_of(i) - prefix_keys : (is_multi(n) ? len_of(i) : 0);
  };
  // Partition length P: the caller's, or chosen here from the step's actual lengths so
  // that the decode-path keys fill about decode_slots (kv head, partition) tasks of equal
  // length: P = keys * Hkv / slots in whole 32-key steps, at least kMinPartTokens, then
  // raised in proportion if the whole-partition rounding of each sequence overshoots the
  // slots. A sequence shorter than P stays whole.
  int P = p.part_tokens;
  if (P == 0) {
    const int64_t keys = 32 * ((int64_t)total[2] + total[3]) - (int64_t)total_dec * prefix_keys;
    const int64_t slots = p.decode_slots;
    int64_t want = (keys * hkv + slots - 1) / slots;
    want = imin64(imax64((want + 31) / 32 * 32, kMinPartTokens), 1 << 30);
    int32_t nt[1] = {0};
    for (int i = b; i < e; ++i) nt[0] += split_parts(task_len(i), (int)want).n;
    int32_t nb[1], ntot[1];
    block_scan_min<1, 0>(red, tid, nt, nb, ntot, nullptr);
    if ((int64_t)ntot[0] * hkv > slots)
      want = imin64((want * ntot[0] * hkv + slots - 1) / slots + 31, 1 << 30) / 32 * 32;
    P = (int)want;
  }
  // Shared-prefix partitions: at least min(P, 512) keys each (a multiple of 64), and at
  // most max(kPrefixSlotRows / decode rows, 1) of them, which bounds the partials.
  int pparts = 0, pplen = 0;
  if (prefix_keys > 0) {
    const int pmin = (min(P, 512) + 63) / 64 * 64;
    int n = (prefix_keys + pmin - 1) / pmin;
    n = min(n, max(1, kPrefixSlotRows / total_dec));
    pplen = ((prefix_keys + n - 1) / n + 63) / 64 * 64;
    pparts = (prefix_keys + pplen - 1) / pplen;
  }
  // Partials of sequence i, in units of Hkv * G slots: nparts * rows (its live columns
  // are rows * G) when its result is split over two or more partitions (shared-prefix
  // ones included), else none.
  auto part_units = [&](int i) -> int {
    const int n = rows_of(i);
    if (n != 1 && !is_multi(n)) return 0;
    const int nparts = (n == 1 ? pparts : 0) + split_parts(task_len(i), P).n;
    return nparts >= 2 ? nparts * n : 0;
  };
  const int64_t unit_slots = (int64_t)hkv * G;
  // Tasks of exactly P keys come first, in sequence order; the others follow in 32 length
  // buckets over (0, min(P, longest table)], longest bucket first.
  const int Pb = (int)imin64(P, (int64_t)MB * kBlock);
  auto bucket = [&](int tlen) { return min(kBuckets - 1, (tlen - 1) * kBuckets / Pb); };
  // A sequence's partitions all hold plen keys but the last, so its tasks fall in at
  // most two buckets: one LDS atomic each, for all of them.
  int32_t tc[3] = {0, 0, 0};  // tasks of exactly P keys, all tasks, partial units
  for (int i = b; i < e; ++i) {
    const int len = task_len(i);
    const PartSplit sp = split_parts(len, P);
    if (sp.n == 0) continue;
    tc[1] += sp.n;
    const int last = len - (sp.n - 1) * sp.plen;
    if (sp.n > 1) {
      if (sp.plen == P) tc[0] += sp.n - 1;
      else atomicAdd(&bcount[bucket(sp.plen)], sp.n - 1);
    }
    if (last == P) ++tc[0];
    else atomicAdd(&bcount[bucket(last)], 1);
    tc[2] += part_units(i);
  }
  int32_t tb[3], tt[3];
  block_scan_min<3, 0>(red, tid, tc, tb, tt, nullptr);  // (its barriers also publish bcount)
  // The host sizes the task list, the decode grid and the partial area from upper bounds
  // over every plan of these sizes, so this cannot overflow; if it ever did, nothing on
  // the decode path runs (its rows stay unwritten) rather than writing past the workspace.
  const int64_t total_slots = tt[2] * unit_slots;
  const bool overflow = total_slots > p.part_capacity || tt[1] > p.max_tasks;
  if (tid == 0) {
    int run = tt[0];
    for (int k = kBuckets - 1; k >= 0; --k) {
      boff[k] = run;
      run += bcount[k];
    }
    p.plan_hdr[kHdrDecTasks] = overflow ? 0 : run;
    p.plan_hdr[kHdrDecSeqs] = total_dec;
    p.plan_hdr[kHdrPrefixKeys] = overflow ? 0 : prefix_keys;
    p.plan_hdr[kHdrPrefixParts] = overflow ? 0 : pparts;
    p.plan_hdr[kHdrPartSlots] = overflow ? -1 : (int)imin64(total_slots, INT32_MAX);
    p.plan_hdr[kHdrPrefixPartTokens] = pplen;
    p.plan_hdr[kHdrPartTokens] = P;
  }
  lds_barrier();
  if (overflow) return;
  int full_run = tb[0];
  int64_t unit_run = tb[2];
  for (int i = b; i < e; ++i) {
    const int len = task_len(i);
    const PartSplit sp = split_parts(len, P);
    if (sp.n > 0) {
      const int n = rows_of(i);
      const int pre_keys = n == 1 ? prefix_keys : 0;
      const int pre_parts = n == 1 ? pparts : 0;
      DecTask task;
      task.seq = i;
      task.row = q0_of(i);
      task.nrows = n;
      task.len = len_of(i);
      task.nparts = pre_parts + sp.n;
      // partition q of the sequence's own range [pre_keys, len) at list position at
      auto put = [&](int at, int q) {
        task.kbeg = pre_keys + q * sp.plen;
        task.kend = min(task.len, task.kbeg + sp.plen);
        task.slot_part = pre_parts + q;
        p.dec_tasks[at] = task;
      };
      const int last = len - (sp.n - 1) * sp.plen;
      if (sp.n > 1) {
        int at;
        if (sp.plen == P) {
          at = full_run;
          full_run += sp.n - 1;
        } else {
          const int bk = bucket(sp.plen);
          at = boff[bk] + atomicAdd(&bfill[bk], sp.n - 1);
        }
        for (int q = 0; q + 1 < sp.n; ++q) put(at + q, q);
      }
      const int bk = bucket(last);
      put(last == P ? full_run++ : boff[bk] + atomicAdd(&bfill[bk], 1), sp.n - 1);
    }
    p.part_base[i] = unit_run * unit_slots;
    unit_run += part_units(i);
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
