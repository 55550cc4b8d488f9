// Device bodies of the slot mapping and the cache write ("reshape_and_cache"), shared by
// their own kernels (slots.hip, scatter.hip) and by the step prologue (plan.hip), which
// runs both beside the planner in one launch.
//
// Slot of a token: the worker builds, for every token of the step, its position and the
// cache slot its K/V go to before the forward pass (hn.213312.xyz restatement of "Inside
// vLLM", section 一, forward pass). Blocks hold 16 tokens (shengyayun.com blog, 关键实现细节
// item 1); slot = block id * 16 + position within the block.
//
// Cache write: each new token's K/V rows go to the slot the slot mapping names
// (restatement section 一: the KV tensors are bound at init and the slot mapping is built
// each step). One unit of work is (group of 16 consecutive tokens, kv head):
//  * keys keep their row layout in the block ([block][head][offset][d]): each key row is
//    one contiguous run, copied in 16-byte pieces by neighbouring lanes;
//  * values are stored dim-major inside a block ([block][head][d][offset]) so that the
//    attention kernels can feed consecutive tokens of one dimension straight into an
//    MFMA operand. A thread takes one dimension of 16 / elem_bytes consecutive tokens
//    (8 bf16 / 4 fp32 = 16 bytes): when those tokens go to consecutive slots of one
//    block, as the tokens of a prefill chunk do, the thread writes them with a single
//    16-byte store; otherwise (a decode token, a block boundary) it stores each element
//    alone.
// A pure bit copy: nothing is converted or rounded.
#pragma once

#include <type_traits>

#include "pa_internal.h"

namespace pa {

constexpr int kWriteGroup = 16;  // tokens per cache-write unit

// Position and slot of token t (0 <= t < num_tokens). Tokens past query_start_loc[S]
// (padding rows) get position 0 and slot -1, which the cache write skips.
__device__ inline int64_t token_slot(const int32_t* __restrict__ block_tables, const int32_t* __restrict__ qsl,
                                     const int32_t* __restrict__ ctx, int32_t num_seqs, int32_t max_blocks,
                                     int64_t t, int32_t& position) {
  position = 0;
  if (num_seqs == 0 || t >= qsl[num_seqs]) return -1;
  const int i = upper_index(qsl, num_seqs, t);
  const int64_t pos = (int64_t)ctx[i] + (t - qsl[i]);
  const int64_t block = block_tables[(int64_t)i * max_blocks + pos / kBlock];
  position = (int32_t)pos;
  return block * kBlock + pos % kBlock;
}

// One cache-write unit: tokens t0 .. t0 + 15 (those below num_tokens) of kv head h, by
// `nthreads` threads numbered `lt`. slot_of(j) gives the slot of token t0 + j.
template <int kElemBytes, class SlotOf>
__device__ inline void write_unit(const uint8_t* __restrict__ k, const uint8_t* __restrict__ v,
                                  uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache, int64_t t0, int h,
                                  int64_t num_tokens, int32_t num_kv_heads, int32_t head_dim, int lt, int nthreads,
                                  SlotOf&& slot_of) {
  constexpr int kUnit = 16 / kElemBytes;  // tokens per 16-byte value store
  const int64_t row_bytes = (int64_t)head_dim * kElemBytes;
  const int chunks = (int)(row_bytes / 16);   // 16-byte pieces per row
  const int items = kWriteGroup * chunks;     // = head_dim * kElemBytes

  // keys: token j of the group, 16-byte piece c of its row
  for (int it = lt; it < items; it += nthreads) {
    const int j = it / chunks;
    const int c = it % chunks;
    const int64_t t = t0 + j;
    if (t >= num_tokens) continue;
    const int64_t slot = slot_of(j);
    if (slot < 0) continue;
    const int64_t block = slot / kBlock;
    const int off = (int)(slot % kBlock);
    const u32x4 w = *reinterpret_cast<const u32x4*>(k + (t * num_kv_heads + h) * row_bytes + c * 16);
    *reinterpret_cast<u32x4*>(k_cache + ((block * num_kv_heads + h) * kBlock + off) * row_bytes + c * 16) = w;
  }

  // values: dimension d of the kUnit tokens of unit u
  using Elem = typename std::conditional<kElemBytes == 2, uint16_t, uint32_t>::type;
  const Elem* __restrict__ vin = reinterpret_cast<const Elem*>(v);
  Elem* __restrict__ vout = reinterpret_cast<Elem*>(v_cache);
  for (int it = lt; it < items; it += nthreads) {
    const int d = it % head_dim;
    const int u = it / head_dim;
    const int64_t tu = t0 + (int64_t)u * kUnit;
    Elem vals[kUnit];
    int64_t s[kUnit];
    bool packed = tu + kUnit <= num_tokens;
#pragma unroll
    for (int e = 0; e < kUnit; ++e) {
      const int64_t t = tu + e;
      s[e] = t < num_tokens ? slot_of(u * kUnit + e) : -1;
      vals[e] = t < num_tokens ? vin[(t * num_kv_heads + h) * head_dim + d] : Elem(0);
    }
    packed = packed && s[0] >= 0 && s[0] % kUnit == 0;
#pragma unroll
    for (int e = 1; e < kUnit; ++e) packed = packed && s[e] == s[0] + e;
    if (packed) {
      u32x4 w;
      if constexpr (kElemBytes == 2) {
#pragma unroll
        for (int x = 0; x < 4; ++x) w[x] = (uint32_t)vals[2 * x] | ((uint32_t)vals[2 * x + 1] << 16);
      } else {
#pragma unroll
        for (int x = 0; x < 4; ++x) w[x] = vals[x];
      }
      const int64_t block = s[0] / kBlock;
      const int off = (int)(s[0] % kBlock);
      *reinterpret_cast<u32x4*>(vout + ((block * num_kv_heads + h) * head_dim + d) * kBlock + off) = w;
    } else {
#pragma unroll
      for (int e = 0; e < kUnit; ++e) {
        if (s[e] < 0) continue;
        const int64_t block = s[e] / kBlock;
        const int off = (int)(s[e] % kBlock);
        vout[((block * num_kv_heads + h) * head_dim + d) * kBlock + off] = vals[e];
      }
    }
  }
}

}  // namespace pa
