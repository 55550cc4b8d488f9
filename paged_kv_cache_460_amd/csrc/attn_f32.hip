// fp32 attention over the mixed step on the vector ALUs (decode and chunk rows alike).
//
// fp32 payloads need fp32 products (the bf16 matrix cores would round the inputs), so
// this path keeps everything on the VALU: one wave per (query row, kv head) walks the
// row's visible keys 64 at a time, with an online softmax per query head. For the dot
// products a lane holds one key, its row read once in 16-byte pieces and used for every
// query head of the group; for the value sum a lane holds one dimension (two for D =
// 128), reading that dimension's 16 tokens of a block (64 contiguous bytes of the
// dim-major value tile) at a time. bf16 steps use the MFMA kernels.
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
    // Scores: lane = key kb + lane. Its key row is read once, 16 bytes at a time, and
    // dotted with every query head of the group (queries from LDS, broadcast reads).
    const int j = kb + lane;
    const bool valid = j <= pos;
    float s[kMaxG];
#pragma unroll
    for (int h = 0; h < kMaxG; ++h) s[h] = -INFINITY;
    if (valid) {
      const int64_t blk = bt[j / kBlock];
      const f32x4* kr = reinterpret_cast<const f32x4*>(kc + ((blk * hkv + g) * kBlock + j % kBlock) * D);
      f32x4 kv[D / 4];
#pragma unroll
      for (int d4 = 0; d4 < D / 4; ++d4) kv[d4] = kr[d4];
#pragma unroll
      for (int h = 0; h < kMaxG; ++h) {
        if (h < G) {
          const f32x4* qh = reinterpret_cast<const f32x4*>(qs + h * D);
          float acc = 0.f;
#pragma unroll
          for (int d4 = 0; d4 < D / 4; ++d4) {
            const f32x4 qv = qh[d4];
            acc = fmaf(qv[0], kv[d4][0], acc);
            acc = fmaf(qv[1], kv[d4][1], acc);
            acc = fmaf(qv[2], kv[d4][2], acc);
            acc = fmaf(qv[3], kv[d4][3], acc);
          }
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
    // Values: lane = dimension (and + 64). Per 16-key block, a dimension's 16 tokens are
    // 64 contiguous bytes of the dim-major value tile, read as four 16-byte pieces; keys
    // past the row's position are removed by select (their slots may hold NaN).
    const int nk = min(64, pos + 1 - kb);
    for (int b0 = 0; b0 < nk; b0 += kBlock) {
      const int64_t blk = bt[(kb + b0) / kBlock];
      const int nv = min(kBlock, nk - b0);
#pragma unroll
      for (int x = 0; x < kPer; ++x) {
        const f32x4* vr = reinterpret_cast<const f32x4*>(vc + ((blk * hkv + g) * D + lane + 64 * x) * kBlock);
        f32x4 vv[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) vv[c] = vr[c];
#pragma unroll
        for (int kk = 0; kk < kBlock; ++kk) {
          const float v = kk < nv ? vv[kk >> 2][kk & 3] : 0.f;
#pragma unroll
          for (int h = 0; h < kMaxG; ++h)
            if (h < G) o[h][x] = fmaf(ps[h * 64 + b0 + kk], v, o[h][x]);
        }
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
