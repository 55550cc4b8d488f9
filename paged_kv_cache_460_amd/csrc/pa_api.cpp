// C entry points of libpa: argument validation, workspace carve-up, kernel sequencing,
// error reporting and optional per-kernel event timing. Declared in include/pa.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "pa_internal.h"

namespace {

thread_local std::string g_last_error;

pa_status fail(pa_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
pa_status fail(pa_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

pa_status hip_fail(hipError_t e, const char* what) {
  return fail(PA_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

// ---- PA_DEBUG index checks ------------------------------------------------------

bool debug_enabled() {
  const char* e = std::getenv("PA_DEBUG");
  return e && e[0] == '1';
}

const char* check_text(int code) {
  switch (code) {
    case pa::kCheckQslStart: return "query_start_loc[0] is not 0";
    case pa::kCheckQslOrder: return "query_start_loc decreases";
    case pa::kCheckQslEnd: return "query_start_loc[S] exceeds num_tokens";
    case pa::kCheckContext: return "context_lens is negative";
    case pa::kCheckSeqLen: return "seq_lens differs from context_lens + query rows";
    case pa::kCheckTableWidth: return "the sequence needs more than max_blocks_per_seq blocks";
    case pa::kCheckBlockId: return "a block id lies outside [0, num_blocks)";
    case pa::kCheckSlotRange: return "the slot lies outside [-1, 16 * num_blocks)";
    case pa::kCheckSlotDuplicate: return "the slot repeats an earlier token's slot";
  }
  return "unknown violation";
}

// Runs `check` (a pa::check_* call filling index and code) when PA_DEBUG=1; returns PA_OK
// if the mode is off or nothing is violated.
template <class F>
pa_status debug_check(hipStream_t stream, const char* what, F&& check) {
  if (!debug_enabled()) return PA_OK;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cap) == hipSuccess && cap != hipStreamCaptureStatusNone)
    return fail(PA_E_UNSUPPORTED, "PA_DEBUG index checks cannot run inside a stream capture");
  int64_t index = -1;
  int code = 0;
  const hipError_t e = check(&index, &code);
  if (e != hipSuccess) return hip_fail(e, "PA_DEBUG index check");
  if (code == 0) return PA_OK;
  return fail(PA_E_INDEX, "PA_DEBUG (%s): %s %lld: %s", what,
              code >= pa::kCheckSlotRange ? "token" : "sequence", (long long)index, check_text(code));
}

int elem_bytes(pa_dtype dt) { return dt == PA_BF16 ? 2 : 4; }

bool valid_dtype(int dt) { return dt == PA_F32 || dt == PA_BF16; }

// ---- per-kernel event timing ----------------------------------------------------

struct Timing {
  std::mutex mu;
  bool enabled = false;
  struct Pending {
    int kind;
    hipEvent_t start, stop;
  };
  std::vector<Pending> pending;
  std::vector<hipEvent_t> pool;
  double total_ms[PA_KERNEL_KIND_COUNT] = {};
  int64_t launches[PA_KERNEL_KIND_COUNT] = {};

  hipEvent_t take() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
};

Timing& timing() {
  static Timing t;
  return t;
}

// Set while this thread records a step graph: launches are then captured without the
// timing events (a graph holds kernels only).
thread_local bool g_capturing = false;

// A step capture may record the prefill kernel on a side stream that forks after the
// planner and joins at the end, so that the graph runs it beside the decode and merge
// kernels: its output rows (the chunk rows) are disjoint from theirs, and both only read
// the caches. Set only while pa_step_graph_create records such a graph.
struct PrefillBranch {
  hipStream_t side = nullptr;
  hipEvent_t planned = nullptr, done = nullptr;
};
thread_local const PrefillBranch* g_prefill_branch = nullptr;

// Set while pa_step_graph_create records a step: the slot-mapping and cache-write calls
// check their arguments and leave them here instead of launching, and the attention call
// makes one launch for both and the planner (pa::launch_step_prologue), which saves two
// kernel boundaries per replay.
struct StepPrologue {
  pa::PrologueArgs a{};
  bool slots = false, cache = false, launched = false;
};
thread_local StepPrologue* g_prologue = nullptr;

// Rows beyond one per sequence from which a step graph runs prefill on a branch. Measured
// on one MI355X, replays of the two graphs alternated in one process: with 3 x 2048 chunk
// rows beside 1664 decode rows the step took 5.092 ms with the branch and 5.136 ms
// without; a batch of 64 decode rows took 10 us longer with it, so steps of decode rows
// or short multi-row sequences stay on one stream.
constexpr int64_t kPrefillBranchRows = 1024;

// Launch `fn` (returns hipError_t), bracketed by events when timing is on.
template <class F>
hipError_t timed(int kind, hipStream_t stream, F&& fn) {
  Timing& t = timing();
  if (!t.enabled || g_capturing) return fn();
  std::lock_guard<std::mutex> lock(t.mu);
  hipEvent_t a = t.take(), b = t.take();
  if (!a || !b) return hipErrorOutOfMemory;
  hipError_t e = hipEventRecord(a, stream);
  if (e != hipSuccess) return e;
  e = fn();
  if (e != hipSuccess) return e;
  e = hipEventRecord(b, stream);
  if (e != hipSuccess) return e;
  t.pending.push_back({kind, a, b});
  return hipSuccess;
}

}  // namespace

namespace pa {

pa_status report(pa_status s, const char* detail) {
  g_last_error = detail;
  return s;
}

int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
    return 256;
  return n;
}

Partitioning choose_partitioning(int32_t num_seqs, int32_t max_blocks, int64_t num_tokens, int32_t num_q_heads,
                                 int32_t num_kv_heads) {
  const int64_t max_len = (int64_t)max_blocks * kBlock;
  int64_t fixed = 0;
  if (const char* env = std::getenv("PA_KV_PARTITION")) {
    const long v = std::strtol(env, nullptr, 10);
    if (v >= 64 && v <= 65536 && v % 64 == 0) fixed = v;
  }
  Partitioning r;
  r.part_tokens = (int32_t)fixed;
  r.num_kv_heads = num_kv_heads;
  // A decode task is one (sequence, partition, kv head) streamed by one wave. Every task
  // pays a start-up latency before it streams, so few long tasks beat many short ones, as
  // long as there are enough of them to draw the full HBM rate: the planner aims for one
  // task per decode wave slot (8 per CU), all about equally long.
  const int64_t slots = (int64_t)device_cus() * 8;
  r.decode_slots = (int32_t)slots;
  // Bounds over every plan of these sizes. A decode-path sequence of len <= max_len keys
  // is cut into ns = ceil(len / plen) <= ceil(len / P) partitions. With P fixed that is
  // at most Q = ceil(max_len / P). With P chosen by the planner, P >= 256 and P >= (sum
  // of lengths) * Hkv / slots, so all sequences together have at most slots / Hkv + S.
  const int64_t G = num_q_heads / num_kv_heads;
  const int64_t rows_max = std::max<int64_t>(1, 16 / G);
  const int64_t seqs = std::min<int64_t>(num_seqs, num_tokens);  // sequences with rows
  const int64_t pmin = fixed ? fixed : kMinPartTokens;
  const int64_t Q = (max_len + pmin - 1) / pmin;
  int64_t tasks = seqs * Q;
  if (!fixed) tasks = std::min<int64_t>(tasks, (slots + num_kv_heads - 1) / num_kv_heads + seqs);
  r.max_tasks = (int32_t)std::min<int64_t>(std::max<int64_t>(tasks, 1), INT32_MAX);
  // Partial slots, in units of Hkv * G slots (one per kv head and column of a decode
  // row). A sequence is merged when its result is split over nparts >= 2 partitions, and
  // then holds nparts * Hkv * rows * G slots:
  //  * its own partitions ns: split two or more ways, it has len > P keys, so ns <
  //    2 len / P; it has at most 16 / G rows (a longer one is a prefill chunk), and all
  //    such rows together are at most T. With P fixed, 2 len / P <= 2 max_len / P; with
  //    P chosen by the planner, the sum of 2 len / P over sequences is at most
  //    2 slots / Hkv;
  //  * a decode row with a shared prefix and a single partition of its own: one unit;
  //  * shared-prefix partitions: the planner keeps (decode rows) x (prefix partitions)
  //    at most max(kPrefixSlotRows, decode rows).
  int64_t own = 0;
  if (Q >= 2) {
    own = Q * std::min<int64_t>(num_tokens, seqs * rows_max);
    own = std::min(own, fixed ? rows_max * ((2 * seqs * max_len + fixed - 1) / fixed)
                              : rows_max * ((2 * slots + num_kv_heads - 1) / num_kv_heads));
  }
  const int64_t prefix = std::max<int64_t>(kPrefixSlotRows, seqs);
  r.part_capacity = (own + seqs + prefix) * G * num_kv_heads;
  return r;
}

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

WorkspaceLayout workspace_layout(int32_t num_seqs, int32_t head_dim, pa_dtype dtype, const Partitioning& part) {
  WorkspaceLayout w{};
  if (dtype != PA_BF16 || num_seqs == 0) return w;  // the fp32 path needs no workspace
  size_t off = 0;
  w.tile_offsets = off;
  off += align256(sizeof(int32_t) * ((size_t)num_seqs + 1));
  w.plan_hdr = off;
  off += align256(sizeof(int32_t) * kHdrSize);
  w.dec_tasks = off;
  off += align256(sizeof(DecTask) * (size_t)part.max_tasks);
  w.dec_seqs = off;
  off += align256(sizeof(int32_t) * (size_t)num_seqs);
  w.part_base = off;
  off += align256(sizeof(int64_t) * (size_t)num_seqs);
  w.part_o = off;
  off += align256((size_t)part.part_capacity * (size_t)head_dim * sizeof(float));
  w.part_ml = off;
  off += align256((size_t)part.part_capacity * 2 * sizeof(float));
  w.total = off;
  return w;
}

}  // namespace pa

extern "C" {

const char* pa_status_string(pa_status s) {
  switch (s) {
    case PA_OK: return "PA_OK";
    case PA_E_NULL: return "PA_E_NULL: required pointer is NULL";
    case PA_E_DTYPE: return "PA_E_DTYPE: unknown dtype";
    case PA_E_SHAPE: return "PA_E_SHAPE: invalid or inconsistent size";
    case PA_E_UNSUPPORTED: return "PA_E_UNSUPPORTED: shape not supported by the library";
    case PA_E_ALIGN: return "PA_E_ALIGN: payload pointer not 16-byte aligned";
    case PA_E_WORKSPACE: return "PA_E_WORKSPACE: workspace missing or too small";
    case PA_E_HIP: return "PA_E_HIP: HIP runtime error";
    case PA_E_NO_SPACE: return "PA_E_NO_SPACE: not enough free KV blocks";
    case PA_E_REQUEST: return "PA_E_REQUEST: unknown or duplicate request, or a call out of order";
    case PA_E_INDEX: return "PA_E_INDEX: an index value breaks a precondition (PA_DEBUG)";
  }
  return "unknown pa_status";
}

const char* pa_last_error(void) { return g_last_error.c_str(); }

int pa_version(void) { return PA_VERSION; }

pa_status pa_build_slot_mapping(const int32_t* block_tables, const int32_t* query_start_loc,
                                const int32_t* context_lens, int32_t num_seqs,
                                int32_t max_blocks_per_seq, int64_t num_tokens, int32_t* positions,
                                int64_t* slot_mapping, void* stream) {
  if (num_seqs < 0 || num_tokens < 0) return fail(PA_E_SHAPE, "num_seqs=%d num_tokens=%lld must be >= 0", num_seqs, (long long)num_tokens);
  if (num_seqs > 0 && max_blocks_per_seq < 1) return fail(PA_E_SHAPE, "max_blocks_per_seq=%d must be >= 1", max_blocks_per_seq);
  if (num_tokens > ((int64_t)1 << 31) * 255) return fail(PA_E_SHAPE, "num_tokens=%lld too large", (long long)num_tokens);
  if (num_tokens == 0) return PA_OK;
  if (!slot_mapping || !query_start_loc) return fail(PA_E_NULL, "slot_mapping and query_start_loc are required");
  if (num_seqs > 0 && (!block_tables || !context_lens)) return fail(PA_E_NULL, "block_tables and context_lens are required");
  const hipStream_t s = static_cast<hipStream_t>(stream);
  // (the block count is not an argument here: only negative block ids are caught)
  const pa_status dc = debug_check(s, "slot mapping", [&](int64_t* index, int* code) {
    return pa::check_step_indices(query_start_loc, context_lens, nullptr, block_tables, num_seqs, max_blocks_per_seq,
                                  num_tokens, INT64_MAX, s, index, code);
  });
  if (dc != PA_OK) return dc;
  if (g_prologue) {
    pa::PrologueArgs& a = g_prologue->a;
    a.block_tables = block_tables;
    a.qsl = query_start_loc;
    a.ctx = context_lens;
    a.num_seqs = num_seqs;
    a.max_blocks = max_blocks_per_seq;
    a.num_tokens = num_tokens;
    a.positions = positions;
    a.slots = slot_mapping;
    g_prologue->slots = true;
    return PA_OK;
  }
  const hipError_t e = timed(PA_KERNEL_SLOT_MAPPING, s, [&] {
    return pa::launch_slot_mapping(block_tables, query_start_loc, context_lens, num_seqs, max_blocks_per_seq,
                                   num_tokens, positions, slot_mapping, s);
  });
  if (e != hipSuccess) return hip_fail(e, "slot mapping launch");
  return PA_OK;
}

pa_status pa_reshape_and_cache(const void* k, const void* v, void* k_cache, void* v_cache,
                               const int64_t* slot_mapping, int64_t num_tokens, int32_t num_kv_heads,
                               int32_t head_dim, int64_t num_blocks, pa_dtype dtype, void* stream) {
  if (!valid_dtype(dtype)) return fail(PA_E_DTYPE, "dtype=%d is not PA_F32 or PA_BF16", (int)dtype);
  if (num_tokens < 0 || num_kv_heads < 1 || head_dim < 1 || num_blocks < 1)
    return fail(PA_E_SHAPE, "num_tokens=%lld num_kv_heads=%d head_dim=%d num_blocks=%lld out of range",
                (long long)num_tokens, num_kv_heads, head_dim, (long long)num_blocks);
  if (head_dim != 64 && head_dim != 128) return fail(PA_E_UNSUPPORTED, "head_dim=%d (64 or 128 supported)", head_dim);
  const int eb = elem_bytes(dtype);
  const int64_t groups = (num_tokens + 15) / 16 * (int64_t)num_kv_heads;  // scatter workgroups
  if (groups > INT32_MAX) return fail(PA_E_SHAPE, "step too large for one launch");
  if (num_tokens == 0) return PA_OK;
  if (!k || !v || !k_cache || !v_cache || !slot_mapping) return fail(PA_E_NULL, "k, v, k_cache, v_cache and slot_mapping are required");
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(PA_E_ALIGN, "k, v, k_cache and v_cache must be 16-byte aligned");
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const pa_status dc = debug_check(s, "cache write", [&](int64_t* index, int* code) {
    return pa::check_slot_indices(slot_mapping, num_tokens, num_blocks, s, index, code);
  });
  if (dc != PA_OK) return dc;
  if (g_prologue) {
    pa::PrologueArgs& a = g_prologue->a;
    if (!g_prologue->slots || a.slots != slot_mapping || a.num_tokens != num_tokens)
      return fail(PA_E_SHAPE, "a recorded step writes the caches with the slot mapping it builds");
    a.k = k;
    a.v = v;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.num_kv_heads = num_kv_heads;
    a.head_dim = head_dim;
    a.elem_bytes = eb;
    g_prologue->cache = true;
    return PA_OK;
  }
  const hipError_t e = timed(PA_KERNEL_SCATTER, s, [&] {
    return pa::launch_scatter(k, v, k_cache, v_cache, slot_mapping, num_tokens, num_kv_heads, head_dim, eb, s);
  });
  if (e != hipSuccess) return hip_fail(e, "scatter launch");
  return PA_OK;
}

static pa_status check_attention_sizes(int32_t num_seqs, int32_t max_blocks_per_seq, int64_t num_tokens,
                                       int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                       int dtype) {
  if (!valid_dtype(dtype)) return fail(PA_E_DTYPE, "dtype=%d is not PA_F32 or PA_BF16", dtype);
  if (num_seqs < 0 || num_tokens < 0) return fail(PA_E_SHAPE, "num_seqs=%d num_tokens=%lld must be >= 0", num_seqs, (long long)num_tokens);
  if (num_seqs > 0 && max_blocks_per_seq < 1) return fail(PA_E_SHAPE, "max_blocks_per_seq=%d must be >= 1", max_blocks_per_seq);
  if (max_blocks_per_seq > (1 << 26)) return fail(PA_E_SHAPE, "max_blocks_per_seq=%d too large", max_blocks_per_seq);
  if (num_q_heads < 1 || num_kv_heads < 1) return fail(PA_E_SHAPE, "head counts must be >= 1");
  if (num_q_heads % num_kv_heads) return fail(PA_E_SHAPE, "num_q_heads=%d is not a multiple of num_kv_heads=%d", num_q_heads, num_kv_heads);
  if (num_q_heads / num_kv_heads > 16) return fail(PA_E_UNSUPPORTED, "group size %d (1..16 supported)", num_q_heads / num_kv_heads);
  if (head_dim != 64 && head_dim != 128) return fail(PA_E_UNSUPPORTED, "head_dim=%d (64 or 128 supported)", head_dim);
  if (num_tokens > (int64_t)INT32_MAX / 2) return fail(PA_E_SHAPE, "num_tokens=%lld too large", (long long)num_tokens);
  return PA_OK;
}

pa_status pa_attention_workspace_size(int32_t num_seqs, int32_t max_blocks_per_seq, int64_t num_tokens,
                                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                      pa_dtype dtype, size_t* bytes) {
  if (!bytes) return fail(PA_E_NULL, "bytes is required");
  const pa_status st = check_attention_sizes(num_seqs, max_blocks_per_seq, num_tokens, num_q_heads,
                                             num_kv_heads, head_dim, dtype);
  if (st != PA_OK) return st;
  const pa::Partitioning part =
      pa::choose_partitioning(num_seqs, max_blocks_per_seq, num_tokens, num_q_heads, num_kv_heads);
  *bytes = pa::workspace_layout(num_seqs, head_dim, dtype, part).total;
  return PA_OK;
}

pa_status pa_attention(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                       const int32_t* seq_lens, const int32_t* query_start_loc, const int32_t* context_lens,
                       float scale, void* out, int32_t num_seqs, int32_t max_blocks_per_seq, int64_t num_tokens,
                       int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks,
                       pa_dtype dtype, void* workspace, size_t workspace_bytes, void* stream) {
  pa_status st = check_attention_sizes(num_seqs, max_blocks_per_seq, num_tokens, num_q_heads, num_kv_heads,
                                       head_dim, dtype);
  if (st != PA_OK) return st;
  if (!std::isfinite(scale)) return fail(PA_E_SHAPE, "scale must be finite");
  if (num_seqs == 0 || num_tokens == 0) return PA_OK;
  if (num_blocks < 1) return fail(PA_E_SHAPE, "num_blocks=%lld must be >= 1", (long long)num_blocks);
  if (!q || !k_cache || !v_cache || !block_tables || !seq_lens || !query_start_loc || !context_lens || !out)
    return fail(PA_E_NULL, "q, k_cache, v_cache, block_tables, seq_lens, query_start_loc, context_lens and out are required");
  if (!aligned16(q) || !aligned16(out) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(PA_E_ALIGN, "q, out, k_cache and v_cache must be 16-byte aligned");

  pa::AttnParams p{};
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.block_tables = block_tables;
  p.seq_lens = seq_lens;
  p.qsl = query_start_loc;
  p.ctx = context_lens;
  p.out = out;
  p.num_seqs = num_seqs;
  p.max_blocks = max_blocks_per_seq;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.head_dim = head_dim;
  p.group = num_q_heads / num_kv_heads;
  p.num_tokens = num_tokens;
  p.num_blocks = num_blocks;
  p.scale = scale;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const pa_status dc = debug_check(s, "attention", [&](int64_t* index, int* code) {
    return pa::check_step_indices(query_start_loc, context_lens, seq_lens, block_tables, num_seqs, max_blocks_per_seq,
                                  num_tokens, num_blocks, s, index, code);
  });
  if (dc != PA_OK) return dc;

  // In a recorded step the slot mapping and cache write run here, in the planner's launch
  // (none for fp32).
  StepPrologue* const pro = g_prologue && g_prologue->cache ? g_prologue : nullptr;
  if (pro) pro->launched = true;

  if (dtype == PA_F32) {
    if (pro) {
      const hipError_t e = pa::launch_step_prologue(pro->a, nullptr, s);
      if (e != hipSuccess) return hip_fail(e, "step prologue launch");
    }
    const hipError_t e = timed(PA_KERNEL_ATTN_F32, s, [&] { return pa::launch_attn_f32(p, s); });
    if (e != hipSuccess) return hip_fail(e, "fp32 attention launch");
    return PA_OK;
  }

  const pa::Partitioning part =
      pa::choose_partitioning(num_seqs, max_blocks_per_seq, num_tokens, num_q_heads, num_kv_heads);
  p.part_tokens = part.part_tokens;
  p.decode_slots = part.decode_slots;
  p.max_tasks = part.max_tasks;
  p.part_capacity = part.part_capacity;
  // The planner counts partials in 32-bit units of Hkv * G slots.
  if (part.part_capacity / ((int64_t)num_q_heads) > INT32_MAX)
    return fail(PA_E_SHAPE, "step too large: %lld partial slots", (long long)part.part_capacity);
  // One decode workgroup per (task, kv head) pair of the task bound; those past the
  // planner's tasks exit at once.
  const int64_t pairs = (int64_t)p.max_tasks * num_kv_heads;
  if (pairs > INT32_MAX) return fail(PA_E_SHAPE, "decode grid of %lld workgroups too large", (long long)pairs);
  p.decode_wgs = (int32_t)pairs;
  const pa::WorkspaceLayout w = pa::workspace_layout(num_seqs, head_dim, dtype, part);
  if (!workspace || workspace_bytes < w.total)
    return fail(PA_E_WORKSPACE, "workspace of %zu bytes needed, %zu given%s", w.total, workspace_bytes,
                workspace ? "" : " (NULL)");
  if (!aligned16(workspace)) return fail(PA_E_ALIGN, "workspace must be 16-byte aligned");
  char* base = static_cast<char*>(workspace);
  p.tile_offsets = reinterpret_cast<int32_t*>(base + w.tile_offsets);
  p.plan_hdr = reinterpret_cast<int32_t*>(base + w.plan_hdr);
  p.dec_tasks = reinterpret_cast<pa::DecTask*>(base + w.dec_tasks);
  p.dec_seqs = reinterpret_cast<int32_t*>(base + w.dec_seqs);
  p.part_base = reinterpret_cast<int64_t*>(base + w.part_base);
  p.part_o = reinterpret_cast<float*>(base + w.part_o);
  p.part_ml = reinterpret_cast<float*>(base + w.part_ml);

  const PrefillBranch* br = g_capturing ? g_prefill_branch : nullptr;
  hipError_t e = timed(PA_KERNEL_PLAN, s, [&] {
    return pro ? pa::launch_step_prologue(pro->a, &p, s) : pa::launch_plan(p, s);
  });
  if (e != hipSuccess) return hip_fail(e, "plan launch");
  if (br) {
    e = hipEventRecord(br->planned, s);
    if (e == hipSuccess) e = hipStreamWaitEvent(br->side, br->planned, 0);
    if (e != hipSuccess) return hip_fail(e, "forking the step graph");
  }
  e = timed(PA_KERNEL_PREFIX, s, [&] { return pa::launch_prefix_bf16(p, s); });
  if (e != hipSuccess) return hip_fail(e, "shared-prefix launch");
  e = timed(PA_KERNEL_DECODE, s, [&] { return pa::launch_decode_bf16(p, s); });
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  e = timed(PA_KERNEL_REDUCE, s, [&] { return pa::launch_reduce(p, s); });
  if (e != hipSuccess) return hip_fail(e, "reduce launch");
  const hipStream_t sf = br ? br->side : s;
  e = timed(PA_KERNEL_PREFILL, sf, [&] { return pa::launch_prefill_bf16(p, sf); });
  if (e == hipSuccess && br) {
    e = hipEventRecord(br->done, sf);
    if (e == hipSuccess) e = hipStreamWaitEvent(s, br->done, 0);
  }
  if (e != hipSuccess) return hip_fail(e, "prefill launch");
  return PA_OK;
}

pa_status pa_attention_plan_info(const void* workspace, size_t workspace_bytes, int32_t num_seqs,
                                 int32_t max_blocks_per_seq, int64_t num_tokens, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim, pa_dtype dtype, int32_t* info,
                                 void* stream) {
  if (!info) return fail(PA_E_NULL, "info is required");
  const pa_status st = check_attention_sizes(num_seqs, max_blocks_per_seq, num_tokens, num_q_heads, num_kv_heads,
                                             head_dim, dtype);
  if (st != PA_OK) return st;
  if (dtype != PA_BF16 || num_seqs == 0 || num_tokens == 0) return PA_OK;  // nothing planned
  const pa::Partitioning part =
      pa::choose_partitioning(num_seqs, max_blocks_per_seq, num_tokens, num_q_heads, num_kv_heads);
  const pa::WorkspaceLayout w = pa::workspace_layout(num_seqs, head_dim, dtype, part);
  if (!workspace || workspace_bytes < w.total)
    return fail(PA_E_WORKSPACE, "workspace of %zu bytes needed, %zu given", w.total, workspace_bytes);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipStreamSynchronize(s);
  if (e == hipSuccess)
    e = hipMemcpy(info, static_cast<const char*>(workspace) + w.plan_hdr, sizeof(int32_t) * pa::kHdrInfo,
                  hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "reading the plan");
  return PA_OK;
}

// ---- step graphs ---------------------------------------------------------------

struct pa_step_graph {
  hipGraph_t graph;
  hipGraphExec_t exec;
};

pa_status pa_step_graph_create(const void* q, const void* k, const void* v, void* k_cache, void* v_cache,
                               const int32_t* block_tables, const int32_t* seq_lens,
                               const int32_t* query_start_loc, const int32_t* context_lens, float scale,
                               void* out, int32_t* positions, int64_t* slot_mapping, int32_t num_seqs,
                               int32_t max_blocks_per_seq, int64_t num_tokens, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks, pa_dtype dtype,
                               void* workspace, size_t workspace_bytes, pa_step_graph** graph) {
  if (!graph) return fail(PA_E_NULL, "graph is required");
  *graph = nullptr;
  // Every check the three calls make is made here first, so a bad argument never opens a capture.
  pa_status st = check_attention_sizes(num_seqs, max_blocks_per_seq, num_tokens, num_q_heads, num_kv_heads,
                                       head_dim, dtype);
  if (st != PA_OK) return st;
  if (num_seqs < 1 || num_tokens < 1 || num_blocks < 1)
    return fail(PA_E_SHAPE, "a step graph needs num_seqs, num_tokens and num_blocks >= 1");
  if (!std::isfinite(scale)) return fail(PA_E_SHAPE, "scale must be finite");
  if (!q || !k || !v || !k_cache || !v_cache || !block_tables || !seq_lens || !query_start_loc || !context_lens ||
      !out || !slot_mapping)
    return fail(PA_E_NULL, "q, k, v, k_cache, v_cache, block_tables, seq_lens, query_start_loc, context_lens, "
                           "out and slot_mapping are required");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache) ||
      !aligned16(out))
    return fail(PA_E_ALIGN, "q, k, v, k_cache, v_cache and out must be 16-byte aligned");
  if (dtype == PA_BF16) {
    const pa::Partitioning part =
        pa::choose_partitioning(num_seqs, max_blocks_per_seq, num_tokens, num_q_heads, num_kv_heads);
    const size_t need = pa::workspace_layout(num_seqs, head_dim, dtype, part).total;
    if (!workspace || workspace_bytes < need)
      return fail(PA_E_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace_bytes);
    if (!aligned16(workspace)) return fail(PA_E_ALIGN, "workspace must be 16-byte aligned");
  }

  hipStream_t cs = nullptr;
  hipError_t e = hipStreamCreateWithFlags(&cs, hipStreamNonBlocking);
  if (e != hipSuccess) return hip_fail(e, "creating the capture stream");
  PrefillBranch br;
  const bool branch = dtype == PA_BF16 && num_tokens - num_seqs >= kPrefillBranchRows;
  auto release = [&] {
    if (br.side) (void)hipStreamDestroy(br.side);
    if (br.planned) (void)hipEventDestroy(br.planned);
    if (br.done) (void)hipEventDestroy(br.done);
    (void)hipStreamDestroy(cs);
  };
  if (branch) {
    e = hipStreamCreateWithFlags(&br.side, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&br.planned, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&br.done, hipEventDisableTiming);
    if (e != hipSuccess) {
      release();
      return hip_fail(e, "creating the prefill branch");
    }
  }
  e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
  if (e != hipSuccess) {
    release();
    return hip_fail(e, "beginning the capture");
  }
  StepPrologue prologue;
  g_capturing = true;
  g_prefill_branch = branch ? &br : nullptr;
  g_prologue = &prologue;
  st = pa_build_slot_mapping(block_tables, query_start_loc, context_lens, num_seqs, max_blocks_per_seq, num_tokens,
                             positions, slot_mapping, cs);
  if (st == PA_OK)
    st = pa_reshape_and_cache(k, v, k_cache, v_cache, slot_mapping, num_tokens, num_kv_heads, head_dim, num_blocks,
                              dtype, cs);
  if (st == PA_OK)
    st = pa_attention(q, k_cache, v_cache, block_tables, seq_lens, query_start_loc, context_lens, scale, out,
                      num_seqs, max_blocks_per_seq, num_tokens, num_q_heads, num_kv_heads, head_dim, num_blocks,
                      dtype, workspace, workspace_bytes, cs);
  g_capturing = false;
  g_prefill_branch = nullptr;
  g_prologue = nullptr;
  if (st == PA_OK && !prologue.launched)
    st = fail(PA_E_SHAPE, "the step's slot mapping and cache write were not launched");
  hipGraph_t g = nullptr;
  e = hipStreamEndCapture(cs, &g);
  release();
  if (st != PA_OK || e != hipSuccess) {
    if (g) (void)hipGraphDestroy(g);
    return st != PA_OK ? st : hip_fail(e, "ending the capture");
  }
  hipGraphExec_t x = nullptr;
  e = hipGraphInstantiate(&x, g, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    (void)hipGraphDestroy(g);
    return hip_fail(e, "instantiating the step graph");
  }
  *graph = new pa_step_graph{g, x};
  return PA_OK;
}

pa_status pa_step_graph_launch(const pa_step_graph* graph, void* stream) {
  if (!graph) return fail(PA_E_NULL, "graph is required");
  const hipError_t e = hipGraphLaunch(graph->exec, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "step graph launch");
  return PA_OK;
}

pa_status pa_step_graph_destroy(pa_step_graph* graph) {
  if (!graph) return PA_OK;
  hipError_t e = hipGraphExecDestroy(graph->exec);
  const hipError_t e2 = hipGraphDestroy(graph->graph);
  delete graph;
  if (e == hipSuccess) e = e2;
  if (e != hipSuccess) return hip_fail(e, "destroying the step graph");
  return PA_OK;
}

pa_status pa_timing_enable(int enable) {
  Timing& t = timing();
  std::lock_guard<std::mutex> lock(t.mu);
  t.enabled = enable != 0;
  return PA_OK;
}

pa_status pa_timing_reset(void) {
  Timing& t = timing();
  std::lock_guard<std::mutex> lock(t.mu);
  for (auto& pd : t.pending) {
    (void)hipEventSynchronize(pd.stop);
    t.pool.push_back(pd.start);
    t.pool.push_back(pd.stop);
  }
  t.pending.clear();
  for (int k = 0; k < PA_KERNEL_KIND_COUNT; ++k) {
    t.total_ms[k] = 0.0;
    t.launches[k] = 0;
  }
  return PA_OK;
}

pa_status pa_timing_read(int kind, double* total_ms, int64_t* launches) {
  if (kind < 0 || kind >= PA_KERNEL_KIND_COUNT) return fail(PA_E_SHAPE, "kernel kind %d out of range", kind);
  if (!total_ms || !launches) return fail(PA_E_NULL, "total_ms and launches are required");
  Timing& t = timing();
  std::lock_guard<std::mutex> lock(t.mu);
  for (auto& pd : t.pending) {
    hipError_t e = hipEventSynchronize(pd.stop);
    if (e != hipSuccess) return hip_fail(e, "timing event");
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, pd.start, pd.stop);
    if (e != hipSuccess) return hip_fail(e, "timing event");
    t.total_ms[pd.kind] += ms;
    t.launches[pd.kind] += 1;
    t.pool.push_back(pd.start);
    t.pool.push_back(pd.stop);
  }
  t.pending.clear();
  *total_ms = t.total_ms[kind];
  *launches = t.launches[kind];
  return PA_OK;
}

}  // extern "C"
