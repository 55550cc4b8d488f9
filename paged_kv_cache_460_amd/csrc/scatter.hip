// Cache write ("reshape_and_cache"): each new token's K/V rows go to the slot the slot
// mapping names (restatement section 一: the KV tensors are bound at init and the
// slot mapping is built each step).
//
// One workgroup per (group of 16 consecutive tokens, kv head).
//  * Keys keep their row layout in the block ([block][head][offset][d]): each key row is
//    one contiguous run, copied in 16-byte pieces by neighbouring lanes.
//  * Values are stored dim-major inside a block ([block][head][d][offset]) so that the
//    attention kernels can feed consecutive tokens of one dimension straight into an
//    MFMA operand. A thread takes one dimension of 16 / elem_bytes consecutive tokens
//    (8 bf16 / 4 fp32 = 16 bytes): when those tokens go to consecutive slots of one
//    block, as the tokens of a prefill chunk do, the thread writes them with a single
//    16-byte store; otherwise (a decode token, a block boundary) it stores each
//    element alone.
// A pure bit copy: nothing is converted or rounded.
#include <type_traits>

#include "pa_internal.h"

namespace pa {

template <int kElemBytes>
__global__ __launch_bounds__(256) void scatter_kernel(
    const uint8_t* __restrict__ k, const uint8_t* __restrict__ v, uint8_t* __restrict__ k_cache,
    uint8_t* __restrict__ v_cache, const int64_t* __restrict__ slots, int64_t num_tokens,
    int32_t num_kv_heads, int32_t head_dim) {
  constexpr int kGroup = 16;                  // tokens per workgroup
  constexpr int kUnit = 16 / kElemBytes;      // tokens per 16-byte value store
  const int h = (int)(blockIdx.x % num_kv_heads);
  const int64_t t0 = (int64_t)(blockIdx.x / num_kv_heads) * kGroup;
  const int64_t row_bytes = (int64_t)head_dim * kElemBytes;
  const int chunks = (int)(row_bytes / 16);   // 16-byte pieces per row
  const int items = kGroup * chunks;          // = head_dim * kElemBytes

  // keys: token j of the group, 16-byte piece c of its row
  for (int it = threadIdx.x; it < items; it += blockDim.x) {
    const int j = it / chunks;
    const int c = it % chunks;
    const int64_t t = t0 + j;
    if (t >= num_tokens) continue;
    const int64_t slot = slots[t];
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
  for (int it = threadIdx.x; it < items; it += blockDim.x) {
    const int d = it % head_dim;
    const int u = it / head_dim;
    const int64_t tu = t0 + (int64_t)u * kUnit;
    Elem vals[kUnit];
    int64_t s[kUnit];
    bool packed = tu + kUnit <= num_tokens;
#pragma unroll
    for (int e = 0; e < kUnit; ++e) {
      const int64_t t = tu + e;
      s[e] = t < num_tokens ? slots[t] : -1;
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

hipError_t launch_scatter(const void* k, const void* v, void* k_cache, void* v_cache,
                          const int64_t* slots, int64_t num_tokens, int32_t num_kv_heads,
                          int32_t head_dim, int32_t elem_bytes, hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const int64_t grid = (num_tokens + 15) / 16 * num_kv_heads;
  if (elem_bytes == 2) {
    hipLaunchKernelGGL(scatter_kernel<2>, dim3((unsigned)grid), dim3(256), 0, stream,
                       (const uint8_t*)k, (const uint8_t*)v, (uint8_t*)k_cache, (uint8_t*)v_cache,
                       slots, num_tokens, num_kv_heads, head_dim);
  } else {
    hipLaunchKernelGGL(scatter_kernel<4>, dim3((unsigned)grid), dim3(256), 0, stream,
                       (const uint8_t*)k, (const uint8_t*)v, (uint8_t*)k_cache, (uint8_t*)v_cache,
                       slots, num_tokens, num_kv_heads, head_dim);
  }
  return hipGetLastError();
}

}  // namespace pa
