// Merge of split-KV decode partials.
//
// Each partition p of a decode row left an unnormalised output o_p, its running max m_p
// (log2 domain) and its weight sum l_p: the shared-prefix partitions (prefill kernel,
// prefix mode) first, then the suffix partitions (decode kernel). Softmax over the
// union of the partitions is
//   out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p,   M = max_p m_p,
// an exact rewrite of the single-pass sum; the result is rounded once to bf16.
// One workgroup per (sequence, kv head) covers that kv head's MFMA columns (a decode
// row's G heads, or up to 16/G rows x G heads of a short multi-row sequence). Its four
// waves take column groups round robin; within a wave D/4 lanes share a column: first
// over partitions for M and the denominator, then over dimensions for the weighted sum,
// eight partitions in flight. A column's partitions sit next to each other, in the
// sequence's region of the partial area (part_slot).
#include "pa_internal.h"

namespace pa {

template <int D>
__global__ __launch_bounds__(256) void reduce_kernel(AttnParams p) {
  constexpr int kLpc = D / 4;      // lanes per column, 4 dims each
  constexpr int kCpw = 64 / kLpc;  // columns per wave pass
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int hkv = p.num_kv_heads;
  const int G = p.group;
  const int i = (int)(blockIdx.x / hkv);
  const int g = (int)(blockIdx.x % hkv);
  const int row0 = p.qsl[i];
  const int nrows = p.qsl[i + 1] - row0;
  const int ncols = nrows * G;
  if (nrows < 1 || ncols > 16 || wave * kCpw >= ncols) return;  // off the decode path, or idle
  if (p.plan_hdr[kHdrPartSlots] < 0) return;  // no plan (see the planner)
  const int P = p.plan_hdr[kHdrPartTokens];
  const int prefix_keys = nrows == 1 ? p.plan_hdr[kHdrPrefixKeys] : 0;
  const int prefix_parts = nrows == 1 ? p.plan_hdr[kHdrPrefixParts] : 0;
  const int nparts = prefix_parts + split_parts(p.seq_lens[i] - prefix_keys, P).n;
  if (nparts <= 1) return;  // the decode kernel wrote the rows itself
  const int cs = lane / kLpc;  // column within the pass
  const int j = lane % kLpc;   // partition stride (max pass), 4-dim group (sum pass)
  const float2* __restrict__ ml = reinterpret_cast<const float2*>(p.part_ml);

  for (int c0 = wave * kCpw; c0 < ncols; c0 += 4 * kCpw) {
    const int c = c0 + cs;
    const bool cvalid = c < ncols;
    const int64_t base = part_slot(p.part_base[i], nparts, ncols, g, cvalid ? c : 0, 0);  // partition q at base + q

    // M = max_q m_q and den = sum_q 2^(m_q - M) l_q, online over this lane's partitions,
    // then merged over the column's lanes. A partition in which a multi-row column saw
    // no key holds m = -inf, l = 0 and adds nothing.
    float M = -INFINITY, den = 0.f;
    if (cvalid) {
      for (int q = j; q < nparts; q += kLpc) {
        const float2 x = ml[base + q];
        const float mn = fmaxf(M, x.x);
        const float mr = mn == -INFINITY ? 0.f : mn;
        den = den * __builtin_amdgcn_exp2f(M - mr) + x.y * __builtin_amdgcn_exp2f(x.x - mr);
        M = mn;
      }
    }
#pragma unroll
    for (int off = kLpc / 2; off > 0; off >>= 1) {
      const float M2 = __shfl_xor(M, off), d2 = __shfl_xor(den, off);
      const float mn = fmaxf(M, M2);
      const float mr = mn == -INFINITY ? 0.f : mn;
      den = den * __builtin_amdgcn_exp2f(M - mr) + d2 * __builtin_amdgcn_exp2f(M2 - mr);
      M = mn;
    }
    if (!cvalid) continue;

    // out = sum_q 2^(m_q - M) o_q / den
    // Loads past the last partition repeat it (clamped index, weight 0), so all eight
    // are issued before the first is used.
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    for (int q0 = 0; q0 < nparts; q0 += 8) {
      float mv[8];
      f32x4 ov[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t slot = base + min(q0 + u, nparts - 1);
        mv[u] = p.part_ml[slot * 2];
        ov[u] = *reinterpret_cast<const f32x4*>(p.part_o + slot * D + j * 4);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float w = q0 + u < nparts ? __builtin_amdgcn_exp2f(mv[u] - M) : 0.f;
        o += w * ov[u];
      }
    }
    const float inv = 1.0f / den;
    uint16_t* orow = static_cast<uint16_t*>(p.out) +
                     ((int64_t)(row0 + c / G) * p.num_q_heads + g * G + c % G) * D + j * 4;
    const u32x2 w = {pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv)};
    *reinterpret_cast<u32x2*>(orow) = w;
  }
}

hipError_t launch_reduce(const AttnParams& p, hipStream_t stream) {
  const int64_t grid = (int64_t)p.num_seqs * p.num_kv_heads;
  if (grid == 0) return hipSuccess;
  if (p.head_dim == 128) {
    hipLaunchKernelGGL(reduce_kernel<128>, dim3((unsigned)grid), dim3(256), 0, stream, p);
  } else {
    hipLaunchKernelGGL(reduce_kernel<64>, dim3((unsigned)grid), dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace pa
