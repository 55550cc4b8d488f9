// Varlen causal prefill on bf16 MFMA (gfx950): the chunks of a mixed step.
//
// Long prompts run in chunks, so a chunk's rows attend to the prompt's cached context
// plus the chunk's own earlier rows (restatement of "Inside vLLM", section 二, item 1;
// shengyayun.com blog, MVP step with the long-prefill threshold). Prefill is the
// compute-bound side of the step (restatement section 一, scheduler), and the only
// dense contraction of the path, so it runs on the matrix cores.
//
// Work unit: (chunk sequence, tile of R rows, kv head). The R rows x G query heads of
// one kv head share every K/V tile, which is staged once in LDS per workgroup:
//  * 4 waves; wave w owns rows [w*RW, (w+1)*RW) of the tile (RW = 32/G) x all G heads,
//    i.e. up to 32 MFMA columns;
//  * keys move in tiles of 64 (4 blocks), gathered through the block table;
//  * S^T = K Q^T and O^T = V^T P^T on 32x32x16 MFMA, so the QK accumulator is already
//    the B operand of PV (see the decode kernel for the same pairing);
//  * online softmax in the log2 domain; causal and end-of-sequence keys are removed by
//    select, and value rows of keys past the sequence end are zeroed when staged, so
//    NaN in unwritten slots cannot leak;
//  * tasks are taken in reverse flat order: last sequence first, last rows first
//    (for the usual ascending-context chunk order, the longest tiles start first);
//  * the kv head is the fastest-varying task index, so with 8 kv heads and a grid that
//    is a multiple of 8, all tiles of one kv head run on one XCD and share its L2.
#include <algorithm>

#include "pa_internal.h"

namespace pa {

namespace {
constexpr float kLog2e = 1.4426950408889634f;
__device__ inline bf16x8 as_bf16x8(u32x4 w) { return __builtin_bit_cast(bf16x8, w); }
}  // namespace

template <int D>
__global__ __launch_bounds__(256) void prefill_bf16_kernel(AttnParams p) {
  constexpr int TK = 64;       // keys per tile (4 blocks)
  constexpr int KS = D + 8;    // LDS row stride of a key row (elements): staggers banks
  constexpr int VS = 20;       // LDS row stride of a value row (16 keys + 4 pad)
  constexpr int KCH = 4 * kBlock * (D / 8);  // 16-byte chunks per key tile
  constexpr int VCH = 4 * D * 2;              // 16-byte chunks per value tile
  static_assert(KCH % 256 == 0 && VCH % 256 == 0, "tile must split evenly over 256 threads");
  __shared__ __attribute__((aligned(16))) uint16_t ks[TK * KS];
  __shared__ __attribute__((aligned(16))) uint16_t vs[4 * D * VS];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 31;   // MFMA column (query row x head)
  const int h2 = lane >> 5;    // lane half
  const int G = p.group;
  const int hkv = p.num_kv_heads;
  const int hq = p.num_q_heads;
  const int RW = 32 / G;
  const int R = 4 * RW;
  const int S = p.num_seqs;
  const int total_tiles = p.tile_offsets[S];
  const int64_t ntasks = (int64_t)total_tiles * hkv;
  const uint16_t* __restrict__ kc = static_cast<const uint16_t*>(p.k_cache);
  const uint16_t* __restrict__ vc = static_cast<const uint16_t*>(p.v_cache);
  const uint16_t* __restrict__ qg = static_cast<const uint16_t*>(p.q);
  uint16_t* __restrict__ og = static_cast<uint16_t*>(p.out);
  const float sl2 = p.scale * kLog2e;

  for (int64_t u = blockIdx.x; u < ntasks; u += gridDim.x) {
    const int g = (int)(u % hkv);
    const int tile = total_tiles - 1 - (int)(u / hkv);
    const int i = upper_index(p.tile_offsets, S, tile);
    const int rt = tile - p.tile_offsets[i];
    const int q0 = p.qsl[i];
    const int n = p.qsl[i + 1] - q0;
    const int ctx = p.ctx[i];
    const int L = p.seq_lens[i];
    const int r0 = rt * R;
    const int kmax = ctx + min(r0 + R, n);  // keys [0, kmax) are seen by some row of the tile
    const int32_t* __restrict__ bt = p.block_tables + (int64_t)i * p.max_blocks;

    const int wr0 = r0 + wave * RW;
    const int wrows = max(0, min(RW, n - wr0));
    const int wkmax = wrows > 0 ? ctx + wr0 + wrows : 0;
    const int crow = wr0 + col / G;
    const bool cvalid = (col < RW * G) && (crow < n);
    const int head = g * G + (col % G);
    const int cpos = cvalid ? ctx + crow : wkmax - 1;

    bf16x8 qb[D / 16];
    {
      const uint16_t* qr = qg + ((int64_t)(q0 + (cvalid ? crow : 0)) * hq + head) * D + h2 * 8;
#pragma unroll
      for (int kq = 0; kq < D / 16; ++kq) {
        const bf16x8 x = *reinterpret_cast<const bf16x8*>(qr + kq * 16);
        qb[kq] = cvalid ? x : bf16x8{};
      }
    }
    f32x16 o[D / 32];
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt) o[mt] = f32x16{};
    float m = -INFINITY;
    float l = 0.f;

    for (int kt = 0; kt < kmax; kt += TK) {
      // ---- gather the tile: 4 blocks of keys and values ----
      u32x4 kreg[KCH / 256], vreg[VCH / 256];
#pragma unroll
      for (int j = 0; j < KCH / 256; ++j) {
        const int chunk = tid + 256 * j;
        const int bl = chunk / (kBlock * (D / 8));
        const int key = (chunk / (D / 8)) % kBlock;
        const int dc = chunk % (D / 8);
        const int b = (kt >> 4) + bl;
        if (b * kBlock < L) {
          const int64_t phys = bt[b];
          kreg[j] = *reinterpret_cast<const u32x4*>(kc + ((phys * hkv + g) * kBlock + key) * D + dc * 8);
        } else {
          kreg[j] = u32x4{0u, 0u, 0u, 0u};
        }
      }
#pragma unroll
      for (int j = 0; j < VCH / 256; ++j) {
        const int chunk = tid + 256 * j;
        const int bl = chunk / (2 * D);
        const int dr = (chunk >> 1) % D;
        const int half = chunk & 1;
        const int b = (kt >> 4) + bl;
        u32x4 w = {0u, 0u, 0u, 0u};
        if (b * kBlock < L) {
          const int64_t phys = bt[b];
          w = *reinterpret_cast<const u32x4*>(vc + ((phys * hkv + g) * D + dr) * kBlock + half * 8);
          const int key0 = b * kBlock + half * 8;
          if (key0 + 8 > L) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (key0 + e >= L) w[e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
          }
        }
        vreg[j] = w;
      }
      __syncthreads();  // every wave is done reading the previous tile
#pragma unroll
      for (int j = 0; j < KCH / 256; ++j) {
        const int chunk = tid + 256 * j;
        const int bl = chunk / (kBlock * (D / 8));
        const int key = (chunk / (D / 8)) % kBlock;
        const int dc = chunk % (D / 8);
        *reinterpret_cast<u32x4*>(&ks[(bl * kBlock + key) * KS + dc * 8]) = kreg[j];
      }
#pragma unroll
      for (int j = 0; j < VCH / 256; ++j) {
        const int chunk = tid + 256 * j;
        const int bl = chunk / (2 * D);
        const int dr = (chunk >> 1) % D;
        const int half = chunk & 1;
        uint16_t* dst = &vs[(bl * D + dr) * VS + half * 8];
        *reinterpret_cast<u32x2*>(dst) = u32x2{vreg[j][0], vreg[j][1]};
        *reinterpret_cast<u32x2*>(dst + 4) = u32x2{vreg[j][2], vreg[j][3]};
      }
      __syncthreads();

      if (kt < wkmax) {
        // ---- S^T = K Q^T for 64 keys x 32 columns ----
        f32x16 s[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          s[mt] = f32x16{};
#pragma unroll
          for (int kq = 0; kq < D / 16; ++kq) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(&ks[(mt * 32 + col) * KS + kq * 16 + h2 * 8]);
            s[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qb[kq], s[mt], 0, 0, 0);
          }
        }
        const bool need_mask = kt + TK - 1 > ctx + wr0;
        float mx = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float x = s[mt][r] * sl2;
            if (need_mask) {
              const int key = kt + mt * 32 + 8 * (r >> 2) + 4 * h2 + (r & 3);
              if (key > cpos) x = -INFINITY;
            }
            s[mt][r] = x;
            mx = fmaxf(mx, x);
          }
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mnew = fmaxf(m, mx);
        const float alpha = __builtin_amdgcn_exp2f(m - mnew);
        float psum = 0.f;
        bf16x8 pb[4];
#pragma unroll
        for (int ub = 0; ub < 4; ++ub) {
          float pe[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            pe[e] = __builtin_amdgcn_exp2f(s[ub >> 1][(ub & 1) * 8 + e] - mnew);
            psum += pe[e];
          }
          const u32x4 w = {pack_bf16x2(pe[0], pe[1]), pack_bf16x2(pe[2], pe[3]),
                           pack_bf16x2(pe[4], pe[5]), pack_bf16x2(pe[6], pe[7])};
          pb[ub] = as_bf16x8(w);
        }
        l = l * alpha + psum;
        m = mnew;
        // ---- O^T += V^T P^T ----
#pragma unroll
        for (int mt = 0; mt < D / 32; ++mt) {
          o[mt] *= alpha;
#pragma unroll
          for (int ub = 0; ub < 4; ++ub) {
            const uint16_t* vr = &vs[(ub * D + mt * 32 + col) * VS + 4 * h2];
            const u32x2 lo = *reinterpret_cast<const u32x2*>(vr);
            const u32x2 hi = *reinterpret_cast<const u32x2*>(vr + 8);
            const u32x4 w = {lo[0], lo[1], hi[0], hi[1]};
            o[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(w), pb[ub], o[mt], 0, 0, 0);
          }
        }
      }
    }
    l += __shfl_xor(l, 32);
    if (cvalid) {
      const float inv = 1.0f / l;
      uint16_t* orow = og + ((int64_t)(q0 + crow) * hq + head) * D + 4 * h2;
#pragma unroll
      for (int mt = 0; mt < D / 32; ++mt) {
#pragma unroll
        for (int grp = 0; grp < 4; ++grp) {
          const u32x2 w = {pack_bf16x2(o[mt][grp * 4 + 0] * inv, o[mt][grp * 4 + 1] * inv),
                           pack_bf16x2(o[mt][grp * 4 + 2] * inv, o[mt][grp * 4 + 3] * inv)};
          *reinterpret_cast<u32x2*>(orow + mt * 32 + grp * 8) = w;
        }
      }
    }
  }
}

hipError_t launch_prefill_bf16(const AttnParams& p, hipStream_t stream) {
  if (p.num_seqs == 0 || p.num_tokens < 2) return hipSuccess;
  const int R = prefill_rows_per_wg(p.group);
  // Upper bound on the tiles the planner can emit: every chunk has >= 2 rows.
  const int64_t chunks = std::min<int64_t>(p.num_seqs, p.num_tokens / 2);
  const int64_t tiles = (p.num_tokens + (int64_t)(R - 1) * chunks) / R + 1;
  int64_t grid = std::min<int64_t>(tiles * p.num_kv_heads, 2048);
  grid = (grid + 7) / 8 * 8;
  if (p.head_dim == 128) {
    hipLaunchKernelGGL(prefill_bf16_kernel<128>, dim3((unsigned)grid), dim3(256), 0, stream, p);
  } else {
    hipLaunchKernelGGL(prefill_bf16_kernel<64>, dim3((unsigned)grid), dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace pa
