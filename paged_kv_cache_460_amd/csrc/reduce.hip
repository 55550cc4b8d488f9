// Merge of split-KV decode partials.
//
// Each partition p of a decode row left an unnormalised output o_p, its running max m_p
// (log2 domain) and its weight sum l_p: the shared-prefix partitions (prefill kernel,
// prefix mode) first, then the suffix partitions (decode kernel). Softmax over the union of the partitions is
//   out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p,   M = max_p m_p,
// an exact rewrite of the single-pass sum; the result is rounded once to bf16.
// One wave per (sequence, query head): lanes take partitions for the max and the
// denominator, then dimensions for the weighted sum (several partitions in flight).
#include "pa_internal.h"

namespace pa {

template <int D>
__global__ __launch_bounds__(256) void reduce_kernel(AttnParams p) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int hq = p.num_q_heads;
  const int64_t item = (int64_t)blockIdx.x * 4 + wave;
  const int i = (int)(item / hq);
  const int h = (int)(item % hq);
  if (i >= p.num_seqs) return;
  const int row = p.qsl[i];
  if (p.qsl[i + 1] - row != 1) return;
  const int P = p.part_tokens;
  const int prefix_keys = p.plan_hdr[kHdrPrefixKeys];
  const int nparts = p.plan_hdr[kHdrPrefixParts] + (p.seq_lens[i] - prefix_keys + P - 1) / P;
  if (nparts <= 1) return;
  const int64_t base = (int64_t)i * p.max_parts * hq + h;  // slot of partition 0; stride hq

  // Pass 1, lanes over partitions: global max M and the denominator sum_p 2^(m_p - M) l_p.
  float M = -INFINITY;
  for (int q = lane; q < nparts; q += 64) M = fmaxf(M, p.part_ml[(base + (int64_t)q * hq) * 2]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  float den = 0.f;
  for (int q = lane; q < nparts; q += 64) {
    const int64_t slot = base + (int64_t)q * hq;
    den += __builtin_amdgcn_exp2f(p.part_ml[slot * 2] - M) * p.part_ml[slot * 2 + 1];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) den += __shfl_xor(den, off);

  // Pass 2, lanes over dims: out = sum_p 2^(m_p - M) o_p / den, 8 partitions in flight.
  constexpr int kPer = D / 64;
  float o[kPer];
#pragma unroll
  for (int x = 0; x < kPer; ++x) o[x] = 0.f;
  for (int q0 = 0; q0 < nparts; q0 += 8) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int q = q0 + u;
      if (q < nparts) {
        const int64_t slot = base + (int64_t)q * hq;
        const float w = __builtin_amdgcn_exp2f(p.part_ml[slot * 2] - M);
        const float* po = p.part_o + slot * D + lane * kPer;
#pragma unroll
        for (int x = 0; x < kPer; ++x) o[x] += w * po[x];
      }
    }
  }
  const float inv = 1.0f / den;
  uint16_t* orow = static_cast<uint16_t*>(p.out) + ((int64_t)row * hq + h) * D + lane * kPer;
  if constexpr (kPer == 2) {
    *reinterpret_cast<uint32_t*>(orow) = pack_bf16x2(o[0] * inv, o[1] * inv);
  } else {
    orow[0] = (uint16_t)f32_to_bf16_bits(o[0] * inv);
  }
}

hipError_t launch_reduce(const AttnParams& p, hipStream_t stream) {
  const int64_t items = (int64_t)p.num_seqs * p.num_q_heads;
  if (items == 0) return hipSuccess;
  const int64_t grid = (items + 3) / 4;
  if (p.head_dim == 128) {
    hipLaunchKernelGGL(reduce_kernel<128>, dim3((unsigned)grid), dim3(256), 0, stream, p);
  } else {
    hipLaunchKernelGGL(reduce_kernel<64>, dim3((unsigned)grid), dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace pa
