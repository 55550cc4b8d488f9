// pa_attention_noalloc: pa_attention with the library's own fixed scratch array as its
// workspace, for callers that cannot allocate device memory (code under stream capture,
// tight serving loops, harnesses that forbid allocation). Declared in include/pa.h.
//
// The scratch is one file-scope device array per GPU, loaded with the code object and
// kept until the process ends. In host code its name is only a host-side stand-in, so
// its device address is looked up once per device (hipGetSymbolAddress, with that device
// current) and that address is what the kernels receive, exactly as they receive a
// caller's workspace. Nothing in it has to start at zero: the planner writes every
// entry the later kernels read, each call. Calls that overlap in time on one GPU share
// the array and race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "pa_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

struct DeviceScratch {
  std::once_flag once;
  hipError_t status = hipSuccess;
  void* ptr = nullptr;
};

DeviceScratch g_scratch[kMaxDevices];

// The scratch array's device address on the current device (looked up on first use).
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  DeviceScratch& d = g_scratch[dev];
  std::call_once(d.once, [&] {
    void* ptr = nullptr;
    d.status = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (d.status == hipSuccess && ptr == nullptr) d.status = hipErrorInvalidSymbol;
    d.ptr = ptr;
  });
  *out = d.ptr;
  return d.status;
}

}  // namespace

extern "C" pa_status pa_attention_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                          const int32_t* block_tables, const int32_t* seq_lens,
                                          const int32_t* query_start_loc, const int32_t* context_lens, float scale,
                                          void* out, int32_t num_seqs, int32_t max_blocks_per_seq,
                                          int64_t num_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                                          int32_t head_dim, int64_t num_blocks, pa_dtype dtype, void* stream) {
  size_t need = 0;
  pa_status st = pa_attention_workspace_size(num_seqs, max_blocks_per_seq, num_tokens, num_q_heads, num_kv_heads,
                                             head_dim, dtype, &need);
  if (st != PA_OK) return st;
  if (need > (size_t)PA_NOALLOC_SCRATCH_BYTES) {
    char msg[200];
    snprintf(msg, sizeof(msg),
             "these sizes need %zu bytes of workspace; the fixed scratch holds %zu (use pa_attention with a "
             "workspace of your own)",
             need, (size_t)PA_NOALLOC_SCRATCH_BYTES);
    return pa::report(PA_E_WORKSPACE, msg);
  }
  void* ws = nullptr;
  if (need > 0) {
    const hipError_t e = scratch_address(&ws);
    if (e != hipSuccess) {
      char msg[200];
      snprintf(msg, sizeof(msg), "looking up the scratch array's device address: %s", hipGetErrorString(e));
      return pa::report(PA_E_HIP, msg);
    }
  }
  return pa_attention(q, k_cache, v_cache, block_tables, seq_lens, query_start_loc, context_lens, scale, out,
                      num_seqs, max_blocks_per_seq, num_tokens, num_q_heads, num_kv_heads, head_dim, num_blocks, dtype,
                      ws, need > 0 ? (size_t)PA_NOALLOC_SCRATCH_BYTES : 0, stream);
}
