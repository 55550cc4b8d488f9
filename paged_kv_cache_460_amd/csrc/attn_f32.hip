// fp32 attention over the mixed step on the vector ALUs (decode and chunk rows alike).
//
// fp32 payloads need fp32 products (the bf16 matrix cores would round the inputs), so
// this path keeps everything on the VALU: one wave per (query row, kv head) walks the
// row's visible keys 64 at a time (one key per lane for the dot products, then one
// dimension slice per lane for the value sum), with an online softmax per query head.
// It is the straightforward path for fp32 steps; bf16 steps use the MFMA kernels.
#include "pa_internal.h"

namespace pa {

namespace {
constexpr float kLog2e = 1.4426950408889634f;

__device__ inline float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ inline float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
}  // namespace

template <int D>
__global__ __launch_bounds__(64) void attn_f32_kernel(AttnParams p) {
  constexpr int kMaxG = 16;
  constexpr int kPer = D / 64;  // dims owned by each lane in the value sum
  __shared__ float qs[kMaxG * D];
  __shared__ float ps[kMaxG * 64];
  const int lane = threadIdx.x;
  const int hkv = p.num_kv_heads;
  const int hq = p.num_q_heads;
  const int G = p.group;
  const int64_t wg = blockIdx.x;
  const int g = (int)(wg % hkv);
  const int64_t t = wg / hkv;
  const int S = p.num_seqs;
  if (S == 0 || t >= p.qsl[S]) return;
  const int i = upper_index(p.qsl, S, t);
  const int pos = p.ctx[i] + (int)(t - p.qsl[i]);
  const float* __restrict__ kc = static_cast<const float*>(p.k_cache);
  const float* __restrict__ vc = static_cast<const float*>(p.v_cache);
  const int32_t* __restrict__ bt = p.block_tables + (int64_t)i * p.max_blocks;
  const float* qrow = static_cast<const float*>(p.q) + (t * hq + g * G) * D;
  for (int x = lane; x < G * D; x += 64) qs[x] = qrow[x];
  __syncthreads();

  const float sl2 = p.scale * kLog2e;
  float o[kMaxG][kPer];
  float m[kMaxG], l[kMaxG];
#pragma unroll
  for (int h = 0; h < kMaxG; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int x = 0; x < kPer; ++x) o[h][x] = 0.f;
  }

  for (int kb = 0; kb <= pos; kb += 64) {
    const int j = kb + lane;
    const bool valid = j <= pos;
    float s[kMaxG];
#pragma unroll
    for (int h = 0; h < kMaxG; ++h) s[h] = -INFINITY;
    if (valid) {
      const int64_t blk = bt[j / kBlock];
      const float* kr = kc + ((blk * hkv + g) * kBlock + j % kBlock) * D;
#pragma unroll
      for (int h = 0; h < kMaxG; ++h) {
        if (h < G) {
          float acc = 0.f;
          for (int d = 0; d < D; ++d) acc = fmaf(qs[h * D + d], kr[d], acc);
          s[h] = acc * sl2;
        }
      }
    }
#pragma unroll
    for (int h = 0; h < kMaxG; ++h) {
      if (h < G) {
        const float mnew = fmaxf(m[h], wave_max(s[h]));
        const float alpha = __builtin_amdgcn_exp2f(m[h] - mnew);
        const float pj = valid ? __builtin_amdgcn_exp2f(s[h] - mnew) : 0.f;
        l[h] = l[h] * alpha + wave_sum(pj);
#pragma unroll
        for (int x = 0; x < kPer; ++x) o[h][x] *= alpha;
        m[h] = mnew;
        ps[h * 64 + lane] = pj;
      }
    }
    __syncthreads();
    const int nk = min(64, pos + 1 - kb);
    for (int jj = 0; jj < nk; ++jj) {
      const int key = kb + jj;
      const int64_t blk = bt[key / kBlock];
      const float* vr = vc + (blk * hkv + g) * D * kBlock + key % kBlock;
#pragma unroll
      for (int x = 0; x < kPer; ++x) {
        const float vv = vr[(int64_t)(lane + 64 * x) * kBlock];
#pragma unroll
        for (int h = 0; h < kMaxG; ++h)
          if (h < G) o[h][x] = fmaf(ps[h * 64 + jj], vv, o[h][x]);
      }
    }
    __syncthreads();
  }
  float* orow = static_cast<float*>(p.out) + (t * hq + g * G) * D;
#pragma unroll
  for (int h = 0; h < kMaxG; ++h) {
    if (h < G) {
      const float inv = 1.0f / l[h];
#pragma unroll
      for (int x = 0; x < kPer; ++x) orow[h * D + lane + 64 * x] = o[h][x] * inv;
    }
  }
}

hipError_t launch_attn_f32(const AttnParams& p, hipStream_t stream) {
  const int64_t grid = p.num_tokens * p.num_kv_heads;
  if (grid == 0 || p.num_seqs == 0) return hipSuccess;
  if (p.head_dim == 128) {
    hipLaunchKernelGGL(attn_f32_kernel<128>, dim3((unsigned)grid), dim3(64), 0, stream, p);
  } else {
    hipLaunchKernelGGL(attn_f32_kernel<64>, dim3((unsigned)grid), dim3(64), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace pa
