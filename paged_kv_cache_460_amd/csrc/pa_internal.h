// Internal declarations shared by the kernels and the C entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

constexpr int kBlock = PA_BLOCK_SIZE;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Query rows handled by one prefill workgroup for group size G (defined beside the
// prefill kernel; the planner cuts chunks into tiles of this many rows).
int prefill_rows_per_tile(int group);

// Everything the attention kernels read; pointers are device pointers.
struct AttnParams {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  const int32_t* qsl;
  const int32_t* ctx;
  void* out;
  int32_t num_seqs;
  int32_t max_blocks;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t group;
  int64_t num_tokens;
  int64_t num_blocks;
  float scale;
  // split-KV decode
  int32_t part_tokens;   // decode partition length P fixed by the caller, or 0: the
                         // planner chooses it from the step's lengths (see plan.hip)
  int32_t decode_slots;  // (kv head, partition) tasks the planner aims to fill
  int32_t max_tasks;     // bound on the planner's decode tasks (task list length)
  int32_t decode_wgs;    // decode workgroups (one wave each): max_tasks * Hkv
  int64_t part_capacity; // partial slots the workspace holds (see choose_partitioning)
  float* part_o;         // [part_capacity, D] unnormalised partial outputs
  float* part_ml;        // [part_capacity, 2] running max (log2 domain) and sum
  // work lists written by the planner
  int32_t* tile_offsets; // [S + 1] exclusive prefix of prefill tiles per sequence
  struct DecTask* dec_tasks;  // [max_tasks] decode tasks, longest first
  int32_t* dec_seqs;     // [S] decode sequences in step order
  int64_t* part_base;    // [S] first partial slot of each sequence that is merged
  int32_t* plan_hdr;     // [kHdrSize] counts and the shared prefix, see kHdr*
};

// One decode task as the planner lists it: one KV partition of a decode row's suffix or
// of a short multi-row sequence, with what a decode wave needs before its first
// block-id load, so that a wave's start-up is a chain of two dependent loads (task, then
// block ids) before it streams keys and values.
struct DecTask {
  int32_t seq;        // sequence index
  int32_t row;        // its first query row (query_start_loc[seq])
  int32_t nrows;      // its query rows: 1, or 2..16/G
  int32_t len;        // its tokens (seq_lens[seq])
  int32_t kbeg, kend; // the task's keys [kbeg, kend)
  int32_t nparts;     // partitions of the sequence's result, shared-prefix ones first
  int32_t slot_part;  // this task's partition among them
};
static_assert(sizeof(DecTask) == 32, "one 32-byte record per task");

// Partials of a sequence whose decode-path result is split over nparts >= 2 partitions
// (shared-prefix partitions first, then its own): one slot per (partition, kv head, live
// MFMA column), in a region of nparts * Hkv * ncols slots that the planner places at
// part_base[i]. The live columns of a kv head are its (row, head-in-group) pairs, c = row
// * G + h % G: ncols = G for a decode row, rows * G (<= 16) for a short multi-row sequence.
// A column's partitions are adjacent, so the merge reads each column's partials in one run.
__host__ __device__ inline int64_t part_slot(int64_t base, int nparts, int ncols, int g, int c, int q) {
  return base + ((int64_t)g * ncols + c) * nparts + q;
}

// Decode-path KV partitions of a range of `len` keys: n partitions of plen keys, the last
// one shorter. plen is len / ceil(len / P) rounded up to whole 32-key steps (never above
// P), so a sequence's partitions are about equally long instead of full P-key ones and a
// short remainder; n <= ceil(len / P), and every partition holds at least one key.
struct PartSplit {
  int n;
  int plen;
};
__host__ __device__ inline PartSplit split_parts(int len, int P) {
  if (len <= 0) return {0, P};
  const int n0 = (len + P - 1) / P;
  int plen = ((len + n0 - 1) / n0 + 31) / 32 * 32;
  plen = plen < P ? plen : P;
  return {(len + plen - 1) / plen, plen};
}

// plan_hdr fields
constexpr int kHdrDecTasks = 0;     // decode tasks in dec_tasks
constexpr int kHdrDecSeqs = 1;      // decode sequences in dec_seqs
constexpr int kHdrPrefixKeys = 2;   // keys of the shared prefix (0: none)
constexpr int kHdrPrefixParts = 3;  // partitions the shared prefix is cut into
constexpr int kHdrPartSlots = 4;    // partial slots the plan uses (<= part_capacity)
constexpr int kHdrPrefixPartTokens = 5;  // keys per shared-prefix partition (multiple of 64)
constexpr int kHdrPartTokens = 6;   // decode partition length P of this plan
constexpr int kHdrSize = 7;
constexpr int kHdrInfo = 7;         // fields reported by pa_attention_plan_info

// Shortest decode partition the planner chooses by itself (a caller may fix a shorter one).
constexpr int kMinPartTokens = 256;

// Shared-prefix partitions: a partition holds at least min(P, 512) keys, and all
// decode rows together hold at most max(kPrefixSlotRows, rows) prefix partials per
// (kv head, column) (one partition each when there are more rows than that): the prefix
// kernel draws its parallelism from the partitions when there are few rows, and from
// the rows when there are many. 512 rather than 1024 halves the partials at 128 rows
// (4096-token prefix: 4 partitions instead of 8) and bounds the prefix grid tighter:
// 64-512 rows on that prefix took 0-7% less time, steps without a prefix the same.
constexpr int kPrefixSlotRows = 512;

// Workspace carve-up (byte offsets from the workspace base).
struct WorkspaceLayout {
  size_t tile_offsets;
  size_t plan_hdr;
  size_t dec_tasks;
  size_t dec_seqs;
  size_t part_base;
  size_t part_o;
  size_t part_ml;
  size_t total;
};

// How a step's decode path is split, as far as the host can know it before the planner
// runs: the partition length if the caller fixes one, and bounds over every plan of the
// call's sizes on the tasks and the partial slots; see choose_partitioning.
struct Partitioning {
  int32_t part_tokens;      // fixed partition length, or 0 (chosen by the planner)
  int32_t decode_slots;     // tasks the planner aims for
  int32_t max_tasks;        // bound on decode tasks
  int64_t part_capacity;    // bound on partial slots
  int32_t num_kv_heads;
};
Partitioning choose_partitioning(int32_t num_seqs, int32_t max_blocks, int64_t num_tokens, int32_t num_q_heads,
                                 int32_t num_kv_heads);
WorkspaceLayout workspace_layout(int32_t num_seqs, int32_t head_dim, pa_dtype dtype, const Partitioning& part);
int device_cus();  // CUs of the current device

// Kernel launchers (defined next to their kernels). Each returns hipGetLastError().
hipError_t launch_slot_mapping(const int32_t* block_tables, const int32_t* qsl, const int32_t* ctx,
                               int32_t num_seqs, int32_t max_blocks, int64_t num_tokens,
                               int32_t* positions, int64_t* slots, hipStream_t stream);
hipError_t launch_scatter(const void* k, const void* v, void* k_cache, void* v_cache,
                          const int64_t* slots, int64_t num_tokens, int32_t num_kv_heads,
                          int32_t head_dim, int32_t elem_bytes, hipStream_t stream);
hipError_t launch_plan(const AttnParams& p, hipStream_t stream);

// Arguments of the slot mapping and the cache write, for the step prologue: one launch
// that builds the slots, writes the caches and, when `plan` is given, runs the planner.
struct PrologueArgs {
  const int32_t* block_tables;
  const int32_t* qsl;
  const int32_t* ctx;
  int32_t num_seqs, max_blocks;
  int64_t num_tokens;
  int32_t* positions;  // may be null
  int64_t* slots;
  const void* k;
  const void* v;
  void* k_cache;
  void* v_cache;
  int32_t num_kv_heads, head_dim, elem_bytes;
};
hipError_t launch_step_prologue(const PrologueArgs& a, const AttnParams* plan, hipStream_t stream);

// PA_DEBUG index checks (debug_checks.hip). Each enqueues its checks on `stream`, waits
// for them and returns the first violation: *code = 0 if none, else one of kCheck*, with
// the sequence (or token) index in *index. seq_lens == nullptr checks the inputs of the
// slot mapping instead of those of attention.
constexpr int kCheckQslStart = 1;       // query_start_loc[0] != 0
constexpr int kCheckQslOrder = 2;       // query_start_loc decreases at sequence i
constexpr int kCheckQslEnd = 3;         // query_start_loc[S] > num_tokens
constexpr int kCheckContext = 4;        // context_lens[i] < 0
constexpr int kCheckSeqLen = 5;         // seq_lens[i] != context_lens[i] + query rows
constexpr int kCheckTableWidth = 6;     // sequence i needs more than max_blocks_per_seq blocks
constexpr int kCheckBlockId = 7;        // a block id sequence i uses lies outside [0, NB)
constexpr int kCheckSlotRange = 8;      // slot_mapping[t] outside [-1, 16 NB)
constexpr int kCheckSlotDuplicate = 9;  // slot_mapping[t] repeats an earlier token's slot
hipError_t check_step_indices(const int32_t* qsl, const int32_t* ctx, const int32_t* seq_lens, const int32_t* bt,
                              int32_t num_seqs, int32_t max_blocks, int64_t num_tokens, int64_t num_blocks,
                              hipStream_t stream, int64_t* index, int* code);
hipError_t check_slot_indices(const int64_t* slots, int64_t num_tokens, int64_t num_blocks, hipStream_t stream,
                              int64_t* index, int* code);

// Set this host thread's pa_last_error() detail and return s (for entry points in other files).
pa_status report(pa_status s, const char* detail);
hipError_t launch_decode_bf16(const AttnParams& p, hipStream_t stream);
hipError_t launch_reduce(const AttnParams& p, hipStream_t stream);
hipError_t launch_prefill_bf16(const AttnParams& p, hipStream_t stream);
hipError_t launch_prefix_bf16(const AttnParams& p, hipStream_t stream);
hipError_t launch_attn_f32(const AttnParams& p, hipStream_t stream);

// --- small device helpers ---------------------------------------------------

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round-to-nearest-even float -> bfloat16 bits (NaN stays NaN).
__device__ inline uint32_t f32_to_bf16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Two floats -> two round-to-nearest-even bfloat16 in one word (lo in bits 0..15);
// a single v_cvt_pk_bf16_f32 on gfx950.
__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// Integer minimum and maximum of 64-bit values. (In device code, min<int64_t>(...) can
// resolve to the floating-point overload, which silently turns later integer divisions
// into exact ones.)
__host__ __device__ inline int64_t imin64(int64_t a, int64_t b) { return a < b ? a : b; }
__host__ __device__ inline int64_t imax64(int64_t a, int64_t b) { return a > b ? a : b; }

// Largest i in [0, n) with a[i] <= x, for non-decreasing a[0..n] and a[0] <= x < a[n].
__device__ inline int upper_index(const int32_t* a, int n, int64_t x) {
  int lo = 0, hi = n;
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (a[mid] <= x) lo = mid; else hi = mid;
  }
  return lo;
}

}  // namespace pa
