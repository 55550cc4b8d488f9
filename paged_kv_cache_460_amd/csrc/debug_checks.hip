// Index checks for PA_DEBUG=1: the preconditions that the fast path takes on trust.
//
// The checks read the index arrays only within their stated sizes and compare values;
// no value is used as an address. A violation is recorded as a key
// (index << 8) | code in a device word, so that the smallest (first) violation wins
// whatever the order in which threads find them. The host reads the word back after
// the checks, with the stream synchronised.
#include <algorithm>

#include "pa_internal.h"

namespace pa {

namespace {

// Smallest violation key seen by the current check; ~0 means none.
__device__ unsigned long long g_first_violation;

__device__ inline void report_violation(int64_t index, int code) {
  atomicMin(&g_first_violation, ((unsigned long long)index << 8) | (unsigned long long)code);
}

__global__ void reset_kernel() { g_first_violation = ~0ull; }

// Per sequence: query offsets, lengths and the block ids its keys use.
__global__ __launch_bounds__(256) void check_steps_kernel(const int32_t* __restrict__ qsl,
                                                          const int32_t* __restrict__ ctx,
                                                          const int32_t* __restrict__ seq_lens,
                                                          const int32_t* __restrict__ bt, int32_t num_seqs,
                                                          int32_t max_blocks, int64_t num_tokens, int64_t num_blocks) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (tid == 0) {
    if (qsl[0] != 0) report_violation(0, kCheckQslStart);
    if ((int64_t)qsl[num_seqs] > num_tokens) report_violation(num_seqs, kCheckQslEnd);
  }
  for (int64_t i = tid; i < num_seqs; i += (int64_t)gridDim.x * blockDim.x) {
    const int n = qsl[i + 1] - qsl[i];
    if (n < 0) {
      report_violation(i, kCheckQslOrder);
      continue;
    }
    if (ctx[i] < 0) {
      report_violation(i, kCheckContext);
      continue;
    }
    if (seq_lens == nullptr) {  // slot-mapping inputs: positions ctx .. ctx + n - 1
      const int64_t need = ((int64_t)ctx[i] + n + kBlock - 1) / kBlock;
      if (need > max_blocks) report_violation(i, kCheckTableWidth);
      for (int64_t j = (int64_t)ctx[i] / kBlock; j < need && j < max_blocks; ++j) {
        const int32_t b = bt[i * max_blocks + j];
        if (b < 0 || b >= num_blocks) {
          report_violation(i, kCheckBlockId);
          break;
        }
      }
      continue;
    }
    const int64_t L = seq_lens[i];
    if (L != (int64_t)ctx[i] + n) {
      report_violation(i, kCheckSeqLen);
      continue;
    }
    const int64_t need = (L + kBlock - 1) / kBlock;
    if (need > max_blocks) {
      report_violation(i, kCheckTableWidth);
      continue;
    }
    for (int64_t j = 0; j < need; ++j) {
      const int32_t b = bt[i * max_blocks + j];
      if (b < 0 || b >= num_blocks) {
        report_violation(i, kCheckBlockId);
        break;
      }
    }
  }
}

// Per token: its slot lies in [-1, 16 NB), and no earlier token has the same non-negative
// slot (quadratic in T: a debugging aid, not a fast path).
__global__ __launch_bounds__(256) void check_slots_kernel(const int64_t* __restrict__ slots, int64_t num_tokens,
                                                          int64_t num_blocks) {
  __shared__ int64_t tile[256];
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t s = t < num_tokens ? slots[t] : -1;
  if (t < num_tokens && (s < -1 || s >= num_blocks * kBlock)) report_violation(t, kCheckSlotRange);
  const int64_t last = (int64_t)blockIdx.x * blockDim.x + blockDim.x;  // tokens before this block's end
  for (int64_t base = 0; base < last && base < num_tokens; base += 256) {
    __syncthreads();
    tile[threadIdx.x] = base + threadIdx.x < num_tokens ? slots[base + threadIdx.x] : -1;
    __syncthreads();
    if (t < num_tokens && s >= 0) {
      const int64_t rem = t - base;
      const int n = rem < 256 ? (int)rem : 256;
      for (int x = 0; x < n; ++x)
        if (tile[x] == s) {
          report_violation(t, kCheckSlotDuplicate);
          break;
        }
    }
  }
}

hipError_t read_first(hipStream_t stream, int64_t* index, int* code) {
  unsigned long long key = ~0ull;
  hipError_t e = hipStreamSynchronize(stream);
  if (e == hipSuccess) e = hipMemcpyFromSymbol(&key, HIP_SYMBOL(g_first_violation), sizeof(key), 0,
                                               hipMemcpyDeviceToHost);
  if (e != hipSuccess) return e;
  *code = key == ~0ull ? 0 : (int)(key & 0xff);
  *index = key == ~0ull ? -1 : (int64_t)(key >> 8);
  return hipSuccess;
}

unsigned grid_for(int64_t n) { return (unsigned)std::max<int64_t>(1, std::min<int64_t>((n + 255) / 256, 1 << 16)); }

}  // namespace

hipError_t check_step_indices(const int32_t* qsl, const int32_t* ctx, const int32_t* seq_lens, const int32_t* bt,
                              int32_t num_seqs, int32_t max_blocks, int64_t num_tokens, int64_t num_blocks,
                              hipStream_t stream, int64_t* index, int* code) {
  hipLaunchKernelGGL(reset_kernel, dim3(1), dim3(1), 0, stream);
  hipLaunchKernelGGL(check_steps_kernel, dim3(grid_for(num_seqs)), dim3(256), 0, stream, qsl, ctx, seq_lens, bt,
                     num_seqs, max_blocks, num_tokens, num_blocks);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return read_first(stream, index, code);
}

hipError_t check_slot_indices(const int64_t* slots, int64_t num_tokens, int64_t num_blocks, hipStream_t stream,
                              int64_t* index, int* code) {
  hipLaunchKernelGGL(reset_kernel, dim3(1), dim3(1), 0, stream);
  const unsigned grid = (unsigned)((num_tokens + 255) / 256);
  if (grid > 0) hipLaunchKernelGGL(check_slots_kernel, dim3(grid), dim3(256), 0, stream, slots, num_tokens, num_blocks);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return read_first(stream, index, code);
}

}  // namespace pa
