/*
 * pa.h -- PagedAttention over a block-paged KV cache, for AMD Instinct MI355X (gfx950).
 *
 * One serving step runs two calls on the caller's HIP stream:
 *
 *   1. pa_reshape_and_cache: write the step's new K/V rows into the block pool at the
 *      slots given by a per-token slot mapping.
 *   2. pa_attention: causal attention for every query row of the step. The rows come
 *      from all scheduled sequences, flattened into one "super-sequence"; decode rows
 *      and chunked-prefill rows are mixed freely. K/V are gathered through each
 *      sequence's block table. Query heads share kv heads in contiguous groups (GQA).
 *
 * Sources (web pages that summarise the article "Inside vLLM: Anatomy of a
 * High-Throughput LLM Inference System"):
 *   - KV cache kept in fixed blocks that are handed out and reclaimed on demand:
 *     chat-gpts.plus news summary, section 事件核心; 16 tokens per block by default:
 *     shengyayun.com "读懂 vLLM 推理引擎内幕", section 关键实现细节, item 1.
 *   - Positions and slot mapping are prepared for each step; all scheduled sequences
 *     are flattened into one super-sequence for a custom paged-attention kernel:
 *     hn.213312.xyz restatement "深入解析 vLLM", section 一, forward pass.
 *   - Decode and prefill mixed in one step; long prompts cut into chunks:
 *     same restatement, section 一 (scheduler) and section 二, item 1.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *   BLOCK   = PA_BLOCK_SIZE = 16 tokens per block.
 *   S       = num_seqs, T = num_tokens, Hq / Hkv = query / kv heads, G = Hq / Hkv,
 *   D       = head_dim, NB = num_blocks, MB = max_blocks_per_seq.
 *   Layouts (all row-major and contiguous; element strides are implied by the shapes):
 *     q, out        [T, Hq, D]
 *     k, v          [T, Hkv, D]            (new rows of this step)
 *     k_cache       [NB, Hkv, BLOCK, D]    k_cache[b][h][o][d] = dim d of the key of the
 *                                          token in slot BLOCK*b + o, kv head h
 *     v_cache       [NB, Hkv, D, BLOCK]    v_cache[b][h][d][o] = dim d of that token's value
 *     block_tables  [S, MB] int32          logical block j of sequence i lives in block
 *                                          block_tables[i][j]; entries at or past
 *                                          ceil(seq_lens[i] / BLOCK) are never read
 *     seq_lens      [S] int32              tokens of sequence i after this step
 *     context_lens  [S] int32              tokens of sequence i cached before this step
 *     query_start_loc [S+1] int32          rows of sequence i are [qsl[i], qsl[i+1]);
 *                                          qsl[0] = 0, non-decreasing, qsl[S] <= T
 *     slot_mapping  [T] int64              slot = BLOCK * block + offset, or -1 = skip
 *   Row r of sequence i is the token at position context_lens[i] + r; it sees keys
 *   0 .. context_lens[i] + r of its sequence. Query head h reads kv head h / G.
 *   Payload dtype is one of pa_dtype and is the same for q, k, v, both caches and out;
 *   all accumulation is fp32.
 *
 * Ownership: every pointer is caller-owned device memory (except pa_*_size outputs,
 * which are host pointers). The library keeps no pointer after a call returns and
 * allocates no device memory in these calls. Device buffers must stay alive until
 * the stream has passed the work.
 *
 * Errors: arguments are validated on the host before anything is enqueued; a non-OK
 * status means nothing was enqueued, and pa_last_error() gives the detail (per host
 * thread). Index values stored in device memory (block ids, slots, lengths) are not
 * checked on the fast path: breaking the preconditions below is undefined behaviour.
 * No C++ exception crosses this interface.
 *
 * Debug mode: with the environment variable PA_DEBUG=1, pa_build_slot_mapping,
 * pa_reshape_and_cache and pa_attention first run a check kernel over the index arrays
 * on the call's stream, wait for it (the call synchronises the stream) and return
 * PA_E_INDEX, with the first violating sequence or token in pa_last_error(), before
 * enqueuing any work. Checked: query_start_loc[0] = 0, non-decreasing, and
 * query_start_loc[S] <= T; context_lens >= 0; seq_lens = context_lens + query rows; the
 * blocks a sequence reads fit in max_blocks_per_seq and their ids lie in [0, NB); slots
 * lie in [-1, 16 NB) and non-negative slots are distinct (a check quadratic in T). The
 * mode cannot run inside a stream capture (PA_E_UNSUPPORTED).
 *
 * Preconditions: non-negative slots are pairwise distinct; seq_lens[i] =
 * context_lens[i] + (qsl[i+1] - qsl[i]); every block id a sequence reads lies in
 * [0, NB); out does not overlap q; k_cache does not overlap v_cache; payload
 * pointers are 16-byte aligned.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_BLOCK_SIZE 16
#define PA_VERSION 1

typedef enum pa_status {
  PA_OK = 0,
  PA_E_NULL = 1,        /* a required pointer is NULL                                  */
  PA_E_DTYPE = 2,       /* unknown payload dtype                                       */
  PA_E_SHAPE = 3,       /* a size is negative, zero where it must not be, or too big   */
  PA_E_UNSUPPORTED = 4, /* valid but not provided: head_dim not 64/128, G not in 1..16 */
  PA_E_ALIGN = 5,       /* a payload pointer is not 16-byte aligned                    */
  PA_E_WORKSPACE = 6,   /* workspace NULL or smaller than pa_attention_workspace_size  */
  PA_E_HIP = 7,         /* the HIP runtime reported an error (launch or event)        */
  PA_E_NO_SPACE = 8,    /* block manager: not enough free KV blocks (nothing changed)  */
  PA_E_REQUEST = 9,     /* block manager: unknown or duplicate request id, or a call
                           that does not fit the request's state                       */
  PA_E_INDEX = 10       /* PA_DEBUG=1: an index value breaks a precondition             */
} pa_status;

typedef enum pa_dtype {
  PA_F32 = 0,  /* IEEE binary32                          */
  PA_BF16 = 1  /* bfloat16 (upper half of a binary32)    */
} pa_dtype;

/* Constant string naming a status. Never NULL. */
const char* pa_status_string(pa_status s);

/* Detail of the last non-OK status returned on this host thread ("" if none). */
const char* pa_last_error(void);

/* PA_VERSION of the built library. */
int pa_version(void);

/*
 * Positions and slot mapping of the step's tokens (the step's index preparation,
 * restatement section 一, forward pass).
 *   positions[t]    = context_lens[i] + (t - qsl[i])        for qsl[i] <= t < qsl[i+1]
 *   slot_mapping[t] = block_tables[i][p / 16] * 16 + p % 16  with p = positions[t]
 * Rows t >= qsl[S] (padding) get position 0 and slot -1.
 * positions may be NULL (not written). block_tables is [S, MB] int32.
 * Errors: PA_E_NULL, PA_E_SHAPE (negative sizes, MB < 1 with S > 0), PA_E_HIP.
 */
pa_status pa_build_slot_mapping(const int32_t* block_tables, const int32_t* query_start_loc,
                                const int32_t* context_lens, int32_t num_seqs,
                                int32_t max_blocks_per_seq, int64_t num_tokens,
                                int32_t* positions, int64_t* slot_mapping, void* stream);

/*
 * Cache write ("reshape_and_cache"): for every t < num_tokens with s = slot_mapping[t] >= 0,
 *   k_cache[s/16][h][s%16][:] = k[t][h][:]   and   v_cache[s/16][h][:][s%16] = v[t][h][:]
 * for all kv heads h. A bit copy: stored bits equal the input bits. Other slots are
 * not touched. Slots must lie in [-1, 16*NB) and be distinct when non-negative.
 * Errors: PA_E_NULL, PA_E_DTYPE, PA_E_SHAPE, PA_E_UNSUPPORTED (D not 64/128),
 * PA_E_ALIGN, PA_E_HIP.
 */
pa_status pa_reshape_and_cache(const void* k, const void* v, void* k_cache, void* v_cache,
                               const int64_t* slot_mapping, int64_t num_tokens,
                               int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks,
                               pa_dtype dtype, void* stream);

/*
 * Bytes of device workspace pa_attention needs for these sizes (written to *bytes).
 * The figure depends only on the arguments (and on PA_KV_PARTITION, see below). It is
 * the planner's work lists plus an area for split-KV partial results sized by an upper
 * bound over every step of these sizes; that bound grows with the sequences that can be
 * split, not with the block-table width (for example 85 MiB for 1667 sequences with
 * tables 513 or 8192 blocks wide, 32 query and 8 kv heads, head_dim 128).
 */
pa_status pa_attention_workspace_size(int32_t num_seqs, int32_t max_blocks_per_seq,
                                      int64_t num_tokens, int32_t num_q_heads,
                                      int32_t num_kv_heads, int32_t head_dim, pa_dtype dtype,
                                      size_t* bytes);

/*
 * Attention over one mixed step. The caches must already hold this step's tokens
 * (call pa_reshape_and_cache first on the same stream). For each row t of sequence i
 * (position p = context_lens[i] + t - qsl[i]) and query head h (kv head g = h / G):
 *   s_j        = scale * dot(q[t][h], K_i[j][g])            for j = 0..p
 *   out[t][h]  = sum_j exp(s_j - max s) V_i[j][g] / sum_j exp(s_j - max s)
 * where K_i[j] / V_i[j] are the key / value of logical token j of sequence i.
 * The result is rounded once to the payload dtype (round to nearest even).
 * Rows t >= qsl[S] of out are not written. Sequences with no rows are skipped.
 * workspace: device memory of at least pa_attention_workspace_size() bytes, 256-byte
 * aligned; its contents on entry do not matter. Calls that share a workspace must
 * not overlap in time.
 * Routing (decided on the device, same results either way): a sequence with one row is a
 * decode row (split-KV decode); a sequence with 2..16/G rows (speculative-decoding
 * verification) also takes the split-KV decode path, its rows side by side with per-row
 * causal limits; a longer sequence is a prefill chunk (MFMA tiles).
 * Decode rows whose sequences all start with the same physical blocks (two or more decode
 * rows; at least 4 whole blocks, holding only cached tokens of every one of them) have
 * that shared prefix attended once for all of them together; the result is the same up
 * to rounding (requests sharing cached prefix blocks: shengyayun.com blog, 关键实现细节
 * item 2).
 * Split-KV partitions: a decode-path range of len keys is cut into ceil(len / P)
 * partitions of about equal length (whole 32-key steps, at most P keys each). The planner
 * chooses P on the device from the step's actual lengths: the decode-path keys times
 * Hkv, spread over one task per decode wave slot of the GPU (8 per CU), in whole 32-key
 * steps and at least 256 keys; a sequence shorter than P stays whole.
 * Environment: PA_KV_PARTITION=<tokens> (a multiple of 64 in [64, 65536]) fixes P instead.
 * Errors: PA_E_NULL, PA_E_DTYPE, PA_E_SHAPE, PA_E_UNSUPPORTED, PA_E_ALIGN,
 * PA_E_WORKSPACE, PA_E_HIP.
 */
pa_status pa_attention(const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_tables, const int32_t* seq_lens,
                       const int32_t* query_start_loc, const int32_t* context_lens, float scale,
                       void* out, int32_t num_seqs, int32_t max_blocks_per_seq,
                       int64_t num_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                       int32_t head_dim, int64_t num_blocks, pa_dtype dtype, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * pa_attention without a workspace argument, for callers that cannot allocate device
 * memory: code under stream capture, tight serving loops, harnesses that forbid
 * allocation. Arguments, results, routing and errors are those of pa_attention (same
 * kernels, bit-identical output); the workspace is instead a fixed device array of
 * PA_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held until the process ends.
 * The call allocates and frees nothing. Sizes whose pa_attention_workspace_size exceeds
 * PA_NOALLOC_SCRATCH_BYTES are rejected with PA_E_WORKSPACE before anything is enqueued
 * (128 MiB holds, for example, 1667 sequences with tables 513 blocks wide, 32 query and
 * 8 kv heads, head_dim 128). All calls on one GPU share that GPU's array and the last
 * call's contents stay in it (nothing in it needs clearing: each call's planner writes
 * what its kernels read), so calls that overlap in time on one GPU, on any streams, race:
 * order them on one stream or with events. The first call on a device looks up the
 * array's device address (PA_E_HIP if that fails).
 * Errors: those of pa_attention, PA_E_WORKSPACE for sizes beyond the scratch.
 */
#define PA_NOALLOC_SCRATCH_BYTES (128u << 20)

pa_status pa_attention_noalloc(const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_tables, const int32_t* seq_lens,
                               const int32_t* query_start_loc, const int32_t* context_lens,
                               float scale, void* out, int32_t num_seqs,
                               int32_t max_blocks_per_seq, int64_t num_tokens, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks,
                               pa_dtype dtype, void* stream);

/*
 * What the on-device planner decided in the last pa_attention call that used this
 * workspace (bf16 steps; the fp32 path plans nothing and leaves info untouched):
 *   info[0] = decode (sequence, KV partition) tasks
 *   info[1] = decode rows (sequences with exactly one query row)
 *   info[2] = keys of the prefix shared by all decode rows and attended once (0: none)
 *   info[3] = partitions that shared prefix was cut into
 *   info[4] = partial-result slots the plan used (one slot = D + 2 floats); the
 *             workspace holds an upper bound over every plan of the call's sizes
 *   info[5] = keys per shared-prefix partition (0: no shared prefix)
 *   info[6] = decode partition length P the plan used
 * The size arguments must be those of that pa_attention call. info is host memory
 * (7 int32). The call waits for `stream` to finish, then copies 28 bytes.
 * Errors: PA_E_NULL, PA_E_DTYPE, PA_E_SHAPE, PA_E_UNSUPPORTED, PA_E_WORKSPACE, PA_E_HIP.
 */
pa_status pa_attention_plan_info(const void* workspace, size_t workspace_bytes, int32_t num_seqs,
                                 int32_t max_blocks_per_seq, int64_t num_tokens,
                                 int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                 pa_dtype dtype, int32_t* info, void* stream);

/*
 * Step graphs: one serving step (pa_build_slot_mapping, pa_reshape_and_cache and
 * pa_attention, in that order) recorded once as a HIP graph and replayed with one launch.
 * Capturing the step's kernels into a graph, to cut the launch overhead of small steps,
 * is what the engine does while it warms up (hn.213312.xyz, section 一, engine start-up;
 * chat-gpts.plus news summary, section 为什么重要).
 *
 * pa_step_graph_create takes the arguments of the three calls (same meaning, layouts and
 * preconditions; positions may be NULL) and records their kernels with these pointers
 * and sizes; nothing runs at creation. The sizes (num_seqs, max_blocks_per_seq,
 * num_tokens, heads, head_dim, num_blocks), the scale, the partition length and every
 * pointer are fixed in the graph. Each replay reads the current contents of the input
 * buffers (q, k, v, block_tables, seq_lens, query_start_loc, context_lens, the caches),
 * so a caller refills them in place between replays; a step with fewer rows fits by
 * padding (rows past query_start_loc[num_seqs] get slot -1 and no output). The graph
 * writes positions (if given), slot_mapping, the caches, out and the workspace: the
 * same writes as the three calls, with the same results. The slot mapping, the cache
 * write and the planner run as one launch in the graph (they are independent of each
 * other, and everything after them needs all three), so a replay crosses two fewer kernel
 * boundaries than the three calls.
 * A bf16 step with num_tokens - num_seqs >= 1024 records the prefill kernel on a graph
 * branch that runs beside the decode and merge kernels (it writes only the chunk rows of
 * out); the results are the same.
 * The graph belongs to the device that was current at creation; launch it on a stream
 * of that device. Replays that share buffers must not overlap in time. Kernel timing
 * (pa_timing_*) does not see kernels run from a graph.
 * Creation errors: PA_E_NULL, PA_E_DTYPE, PA_E_SHAPE (also num_seqs, num_tokens or
 * num_blocks < 1), PA_E_UNSUPPORTED, PA_E_ALIGN, PA_E_WORKSPACE, PA_E_HIP; on error
 * *graph is NULL and nothing was recorded or launched. pa_step_graph_launch returns
 * PA_E_NULL for a NULL graph, else PA_E_HIP on a launch error. pa_step_graph_destroy
 * frees the graph (NULL is a no-op); the caller owns it until then.
 */
typedef struct pa_step_graph pa_step_graph;

pa_status pa_step_graph_create(const void* q, const void* k, const void* v, void* k_cache,
                               void* v_cache, const int32_t* block_tables, const int32_t* seq_lens,
                               const int32_t* query_start_loc, const int32_t* context_lens,
                               float scale, void* out, int32_t* positions, int64_t* slot_mapping,
                               int32_t num_seqs, int32_t max_blocks_per_seq, int64_t num_tokens,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                               int64_t num_blocks, pa_dtype dtype, void* workspace,
                               size_t workspace_bytes, pa_step_graph** graph);
pa_status pa_step_graph_launch(const pa_step_graph* graph, void* stream);
pa_status pa_step_graph_destroy(pa_step_graph* graph);

/*
 * Measurement support. While enabled, every kernel the library launches is bracketed
 * by HIP events on its stream. pa_timing_read waits for the recorded events and returns
 * the summed duration (ms) and the launch count of one kernel kind since the last reset.
 * Kernel kinds: see pa_kernel_kind. Not for concurrent use from several host threads.
 */
typedef enum pa_kernel_kind {
  PA_KERNEL_SLOT_MAPPING = 0,
  PA_KERNEL_SCATTER = 1,
  PA_KERNEL_PLAN = 2,
  PA_KERNEL_DECODE = 3,
  PA_KERNEL_REDUCE = 4,
  PA_KERNEL_PREFILL = 5,
  PA_KERNEL_ATTN_F32 = 6,
  PA_KERNEL_PREFIX = 7,
  PA_KERNEL_KIND_COUNT = 8
} pa_kernel_kind;

pa_status pa_timing_enable(int enable);
pa_status pa_timing_reset(void);
pa_status pa_timing_read(int kind, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
