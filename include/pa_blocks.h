/*
 * pa_blocks.h — host-side KV block manager (C ABI, CPU only).
 *
 * The bookkeeping step before the attention path: it hands out the pool's fixed
 * 16-token KV blocks to requests, reuses cached prefix blocks, and writes the arrays
 * pa_reshape_and_cache / pa_attention read (block tables, lengths, query offsets and
 * the slot mapping). It runs on the host; no call touches a GPU.
 *
 * Sources (web pages that summarise the article "Inside vLLM: Anatomy of a
 * High-Throughput LLM Inference System"):
 *   - the KV-cache manager keeps a queue of free blocks: hn.213312.xyz, "深入解析 vLLM",
 *     section 一, engine construction;
 *   - allocate_slots works out and allocates the blocks a step needs; when blocks run
 *     out the scheduler preempts: same page, section 一, scheduler;
 *   - prefix caching splits a prefix's KV into blocks stored under their hashes, so a
 *     later request reuses them: same page, section 二, item 2;
 *   - each request is hashed per 16-token block (a built-in hash by default, SHA-256
 *     against collisions); the longest cache hit is found by walking the hash-to-block
 *     map block by block; reuse is block aligned, so a partial last block is not
 *     reused: shengyayun.com "读懂 vLLM 推理引擎内幕", section 关键实现细节, items 1 and 2.
 *
 * Policy (fixed, so results are reproducible):
 *   - Blocks 0..N-1 start in the free queue in id order. Allocation takes blocks from
 *     the queue's head; a block that comes back goes to its tail.
 *   - Block j of a request (tokens 16j..16j+15) is "full" once all 16 of its tokens
 *     are known and covered by allocate_slots. With prefix caching on, a full block
 *     gets the hash H(hash of block j-1, its 16 token ids), and the map from hash to
 *     block records it unless that hash already names another block. Block 0's parent
 *     is all zero bytes.
 *   - A request's cache hit is its longest run of leading full blocks whose hashes are
 *     in the map, capped at (num_tokens - 1) / 16 blocks so that at least one token is
 *     computed. Hit blocks are claimed at once: their reference count goes up, and a
 *     hit block with no other holder leaves the free queue.
 *   - A freed request drops one reference on each of its blocks. Blocks left with no
 *     holder go to the free queue's tail, the request's last block first, so a
 *     sequence's tail is reused before its prefix. A cached block keeps its hash while
 *     it waits in the queue. When it is taken for a new allocation, its hash leaves the
 *     map (eviction).
 *
 * Hashes (pa_block_hash): PA_HASH_FNV1A64 is 64-bit FNV-1a over the bytes
 * parent(8) || tokens(16 x int32 little-endian); PA_HASH_SHA256 is SHA-256 (FIPS
 * 180-4) over parent(32) || tokens(64 bytes). A hash value is stored in 32 bytes; an
 * FNV-1a value sits in bytes 0..7, little-endian, with bytes 8..31 zero.
 *
 * Ownership and errors: all pointers are host memory owned by the caller; the manager
 * copies what it keeps. A non-OK status leaves the manager unchanged, and
 * pa_last_error() gives the detail. One manager must not be used from several threads
 * at once.
 */
#ifndef PA_BLOCKS_H
#define PA_BLOCKS_H

#include <stddef.h>
#include <stdint.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_block_hash {
  PA_HASH_FNV1A64 = 0,
  PA_HASH_SHA256 = 1
} pa_block_hash;

typedef struct pa_block_manager pa_block_manager;

/* A manager over num_blocks (>= 1) blocks. prefix_caching: 0 or 1.
 * Errors: PA_E_NULL (bm), PA_E_SHAPE (num_blocks < 1), PA_E_DTYPE (unknown hash). */
pa_status pa_bm_create(int32_t num_blocks, int32_t prefix_caching, pa_block_hash hash,
                       pa_block_manager** bm);
/* Frees the manager; NULL is a no-op. */
pa_status pa_bm_destroy(pa_block_manager* bm);

/* Registers request_id with its num_tokens (>= 1) prompt tokens and claims its cache
 * hit (policy above); *num_cached_tokens (may be NULL) receives 16 x hit blocks. Those
 * tokens count as computed.
 * Errors: PA_E_NULL, PA_E_SHAPE, PA_E_REQUEST (id already registered). */
pa_status pa_bm_add_request(pa_block_manager* bm, int64_t request_id, const int32_t* token_ids,
                            int64_t num_tokens, int64_t* num_cached_tokens);

/* Appends num_tokens (>= 1) generated tokens to the request's known tokens.
 * Errors: PA_E_NULL, PA_E_SHAPE, PA_E_REQUEST (unknown id). */
pa_status pa_bm_append_tokens(pa_block_manager* bm, int64_t request_id, const int32_t* token_ids,
                              int64_t num_tokens);

/* allocate_slots: makes room for the request's next num_new_tokens (>= 1) tokens,
 * positions computed .. computed + num_new_tokens - 1, which must all be known. Takes
 * ceil((computed + num_new_tokens) / 16) minus held blocks from the free queue's head
 * (evicting their old hashes), then hashes the blocks this makes full.
 * Errors: PA_E_REQUEST (unknown id, or tokens not known yet), PA_E_SHAPE,
 * PA_E_NO_SPACE (the free queue is too short; nothing changed: the caller may free, that
 * is preempt, another request and retry). */
pa_status pa_bm_allocate_slots(pa_block_manager* bm, int64_t request_id, int64_t num_new_tokens);

/* Releases the request's blocks (policy above) and forgets the request.
 * Errors: PA_E_REQUEST (unknown id). */
pa_status pa_bm_free_request(pa_block_manager* bm, int64_t request_id);

/* Writes one step's arrays for num_seqs requests, in order, each scheduling its next
 * query_lens[i] (>= 0) tokens, which allocate_slots must already cover:
 *   block_tables [num_seqs, max_blocks_per_seq] int32: the request's blocks, then 0;
 *   context_lens [num_seqs]: computed tokens before the step; seq_lens = context_lens +
 *   query_lens; query_start_loc [num_seqs + 1]: running sum of query_lens;
 *   slot_mapping [num_tokens] int64: 16 x block + offset of each scheduled token, in
 *   row order, then -1 up to num_tokens (padding).
 * Then advances each request's computed count by its query length. num_tokens must be
 * at least the sum of query_lens; a request may appear once.
 * Errors: PA_E_NULL, PA_E_SHAPE (sizes, a request holding more than max_blocks_per_seq
 * blocks, num_tokens too small), PA_E_REQUEST (unknown or repeated id, or query tokens
 * not covered by allocate_slots). */
pa_status pa_bm_build_step(pa_block_manager* bm, const int64_t* request_ids, const int64_t* query_lens,
                           int32_t num_seqs, int32_t max_blocks_per_seq, int32_t* block_tables,
                           int32_t* seq_lens, int32_t* query_start_loc, int32_t* context_lens,
                           int64_t* slot_mapping, int64_t num_tokens);

/* Free-queue length, and the number of hashes in the prefix-cache map.
 * Errors: PA_E_NULL. */
pa_status pa_bm_num_free_blocks(const pa_block_manager* bm, int32_t* num_free);
pa_status pa_bm_num_cached_blocks(const pa_block_manager* bm, int32_t* num_cached);

/* The request's block ids in order (at most `capacity` written; *num_blocks gets the
 * full count) and info[4] = {known tokens, computed tokens, cache-hit tokens, blocks}.
 * Errors: PA_E_NULL, PA_E_REQUEST (unknown id). */
pa_status pa_bm_request_blocks(const pa_block_manager* bm, int64_t request_id, int32_t* blocks,
                               int32_t capacity, int32_t* num_blocks);
pa_status pa_bm_request_info(const pa_block_manager* bm, int64_t request_id, int64_t* info);

/* Reference count of a block, and its free-queue position (-1 if held).
 * Errors: PA_E_NULL, PA_E_SHAPE (block out of range). */
pa_status pa_bm_block_state(const pa_block_manager* bm, int32_t block, int32_t* ref_count,
                            int32_t* free_position);

/* The block hash above, for one block: parent (32 bytes; NULL = zeros), 16 token ids,
 * out (32 bytes). Errors: PA_E_NULL, PA_E_DTYPE (unknown hash). */
pa_status pa_block_hash_compute(pa_block_hash hash, const uint8_t* parent, const int32_t* tokens,
                                uint8_t* out);

#ifdef __cplusplus
}
#endif

#endif /* PA_BLOCKS_H */
