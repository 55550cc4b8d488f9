// Split-KV decode attention on bf16 MFMA (gfx950).
//
// Decode is bound by memory bandwidth, prefill by compute (restatement of "Inside vLLM",
// section 一, scheduler; shengyayun.com blog, 适用场景 and 关键实现细节 item 4). A decode
// row reads every cached K/V byte of its sequence once, so this kernel is built to
// stream whole 16-token blocks from HBM at full rate:
//
//  * one wave = one (sequence, kv partition, kv head), taken in the planner's
//    longest-first order; a sequence's range is cut into ceil(len / P) partitions of
//    about equal length (split_parts). All G query heads of the kv head ride in the N
//    dimension of one 16x16x32 MFMA, so each K/V byte is read once for the whole GQA
//    group (columns past G are zero and ignored);
//  * transposed products: S^T = K Q^T (A = 16 keys x 32 dims straight from the block's
//    token-major key rows, 16 contiguous bytes per lane) and O^T = V^T P^T, where the
//    QK accumulator already holds P^T in the B-operand layout, and the dim-major value
//    block gives each lane 2 x 8 contiguous bytes of V^T (4 keys of block 0, 4 of block 1);
//  * two blocks (32 keys) per step from two operand buffers in turn: the next step's
//    loads are in flight while the current one computes. Every step issues the same
//    loads (past the range the second block repeats the first, masked), which keeps the
//    compiler's wait counts exact: a step waits only for loads issued a step earlier;
//  * online softmax in the log2 domain (scale * log2 e folded once), max/sum over the
//    four lane groups by cross-lane shuffles;
//  * masked keys are removed by select (-inf score, zeroed value), never by multiplying,
//    so unwritten slots that hold NaN cannot leak;
//  * a sequence with a single partition writes its output row directly; otherwise the
//    wave writes (o, m, l) partials and pa::reduce merges them. (Merging in the decode
//    wave that finishes a sequence's last partition needs a device-scope release and
//    acquire per wave, which here write back and invalidate the L2: decode took twice
//    as long on a 64-row batch, so the merge stays a launch of its own.)
#include "pa_internal.h"

namespace pa {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

template <int D>
struct DecodeStep {
  bf16x8 k0[D / 32], k1[D / 32];   // A operands: keys of block 0 / block 1
  u32x2 v0[D / 16], v1[D / 16];    // halves of the V^T A operands
};

__device__ inline bf16x8 as_bf16x8(u32x4 w) { return __builtin_bit_cast(bf16x8, w); }

// Value rows are read once per decode row and each load covers whole 128-byte lines
// (16 dims x 32 bytes): non-temporal (streaming) loads raise the sustained HBM read rate
// for them. Key loads stay ordinary: one MFMA operand covers only half of each line,
// and the other half is read by the next load from the cache.
__device__ inline u32x2 stream_load_u32x2(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
}

// Both blocks of a step; past the range the second block repeats the first (valid memory,
// masked), so every step issues the same loads and the compiler's wait counts stay exact.
template <int D>
__device__ inline void load_step(DecodeStep<D>& s, const uint16_t* __restrict__ kc,
                                 const uint16_t* __restrict__ vc, const int32_t* __restrict__ bt,
                                 int kb, int kend, int hkv, int g, int c, int qd) {
  const int b0 = kb >> 4;
  const int64_t p0 = bt[b0];
  const int64_t p1 = kb + kBlock < kend ? (int64_t)bt[b0 + 1] : p0;
  const uint16_t* kr0 = kc + ((p0 * hkv + g) * kBlock + c) * D + qd * 8;
  const uint16_t* vr0 = vc + ((p0 * hkv + g) * D + c) * kBlock + qd * 4;
  const uint16_t* kr1 = kc + ((p1 * hkv + g) * kBlock + c) * D + qd * 8;
  const uint16_t* vr1 = vc + ((p1 * hkv + g) * D + c) * kBlock + qd * 4;
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) s.k0[kk] = *reinterpret_cast<const bf16x8*>(kr0 + kk * 32);
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) s.v0[dt] = stream_load_u32x2(vr0 + dt * 16 * kBlock);
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) s.k1[kk] = *reinterpret_cast<const bf16x8*>(kr1 + kk * 32);
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) s.v1[dt] = stream_load_u32x2(vr1 + dt * 16 * kBlock);
}

}  // namespace

template <int D>
// Two waves per SIMD: the register allocator must fit both operand buffers in 256 registers.
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void decode_bf16_kernel(AttnParams p) {
  const int lane = threadIdx.x;
  const int c = lane & 15;   // MFMA column: query head g*G + c
  const int qd = lane >> 4;  // lane group: dims qd*8.. of each 32-dim chunk; keys 4qd.. of each block
  const int hkv = p.num_kv_heads;
  // Workgroup -> (task from the planner's longest-first list, kv head); kv head fastest,
  // so the Hkv workgroups of a task read neighbouring 4 KB tiles of the same blocks.
  const int64_t wg = blockIdx.x;
  const int g = (int)(wg % hkv);
  const int64_t t = wg / hkv;
  // A task is one KV partition of a decode row or of a short multi-row sequence
  // (speculative-decoding verification: 2..16/G rows), whose (row, head) pairs fill the
  // MFMA columns. With a shared prefix a decode row covers only its suffix; the prefix
  // partials occupy its first partial slots. The record is read before the task count
  // is checked (every slot up to the grid's bound is in the list's memory), so that the
  // two loads overlap.
  const DecTask task = p.dec_tasks[t];
  if (t >= p.plan_hdr[kHdrDecTasks]) return;
  const int i = task.seq;
  const int row = task.row;
  const int L = task.len;
  const int G = p.group;
  const int hq = p.num_q_heads;
  const int nrows = task.nrows;
  const int kbeg = task.kbeg;
  const int kend = task.kend;
  const int nparts = task.nparts;
  const int slot_part = task.slot_part;
  // the sequence's partial base, loaded now rather than behind the loop (the planner
  // writes it for every sequence)
  const int64_t pbase = p.part_base[i];
  // column c = (row r, head-in-group hh); row r sits at position L - nrows + r and sees
  // keys up to it (causal), so its keys stop at climit
  const int cr = c / G, chh = c % G;
  const bool cvalid = c < nrows * G;
  const int climit = cvalid ? min(kend, L - nrows + cr + 1) : kend;
  const int kmask = min(kend, L - nrows + 1);  // first key some column must not see

  const uint16_t* __restrict__ kc = static_cast<const uint16_t*>(p.k_cache);
  const uint16_t* __restrict__ vc = static_cast<const uint16_t*>(p.v_cache);
  const int32_t* __restrict__ bt = p.block_tables + (int64_t)i * p.max_blocks;

  // B operand Q^T: column c, dims kk*32 + qd*8 .. +8.
  bf16x8 qb[D / 32];
  {
    const uint16_t* qr = static_cast<const uint16_t*>(p.q) +
                         ((int64_t)(row + (cvalid ? cr : 0)) * hq + g * G + (cvalid ? chh : 0)) * D + qd * 8;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
      bf16x8 x = *reinterpret_cast<const bf16x8*>(qr + kk * 32);
      qb[kk] = cvalid ? x : bf16x8{};
    }
  }

  f32x4 acc[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY;
  float lsum = 0.f;
  const float sl2 = p.scale * kLog2e;

  // One step: the 32 keys from kb, operands in cur; updates m, lsum and acc.
  auto step = [&](const DecodeStep<D>& cur, int kb) {
    // S^T for the two blocks: lane holds keys 4qd..4qd+3 of each block, column c.
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur.k0[kk], qb[kk], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur.k1[kk], qb[kk], s1, 0, 0, 0);
    }
    float sv[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sv[e] = s0[e] * sl2;
      sv[4 + e] = s1[e] * sl2;
    }
    const bool tail = kb + 2 * kBlock > kmask;
    uint32_t vmask[4] = {0xffffffffu, 0xffffffffu, 0xffffffffu, 0xffffffffu};
    if (tail) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int key = kb + (e >> 2) * kBlock + 4 * qd + (e & 3);
        if (key >= climit) sv[e] = -INFINITY;
        if (key >= kend) vmask[e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
      }
    }
    float mx = sv[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sv[e]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mnew = fmaxf(m, mx);
    // A multi-row column can see no key at all in a late partition (its row lies
    // before the partition): keep its state at m = -inf, l = 0, o = 0 (weight 0 in the
    // merge) instead of forming -inf - -inf.
    const float mref = mnew == -INFINITY ? 0.f : mnew;
    const float alpha = __builtin_amdgcn_exp2f(m - mref);
    float pe[8];
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pe[e] = __builtin_amdgcn_exp2f(sv[e] - mref);
      psum += pe[e];
    }
    lsum = lsum * alpha + psum;
    m = mnew;
    const u32x4 pw = {pack_bf16x2(pe[0], pe[1]), pack_bf16x2(pe[2], pe[3]),
                      pack_bf16x2(pe[4], pe[5]), pack_bf16x2(pe[6], pe[7])};
    const bf16x8 pb = as_bf16x8(pw);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      u32x4 vw = {cur.v0[dt][0], cur.v0[dt][1], cur.v1[dt][0], cur.v1[dt][1]};
      if (tail) {
        vw[0] &= vmask[0];
        vw[1] &= vmask[1];
        vw[2] &= vmask[2];
        vw[3] &= vmask[3];
      }
      acc[dt] *= alpha;
      acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vw), pb, acc[dt], 0, 0, 0);
    }
  };

  // Two operand buffers in turn, each step the same loads: the next step's loads go out
  // before the current step computes, and the current step waits only for loads issued
  // one step earlier.
  DecodeStep<D> sa, sb;
  load_step<D>(sa, kc, vc, bt, kbeg, kend, hkv, g, c, qd);
  for (int kb = kbeg;;) {
    if (kb + 2 * kBlock < kend) {
      load_step<D>(sb, kc, vc, bt, kb + 2 * kBlock, kend, hkv, g, c, qd);
      step(sa, kb);
    } else {
      step(sa, kb);
      break;
    }
    kb += 2 * kBlock;
    if (kb + 2 * kBlock < kend) {
      load_step<D>(sa, kc, vc, bt, kb + 2 * kBlock, kend, hkv, g, c, qd);
      step(sb, kb);
    } else {
      step(sb, kb);
      break;
    }
    kb += 2 * kBlock;
  }
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);

  if (!cvalid) return;
  const int h = g * G + chh;
  if (nparts == 1) {
    const float inv = 1.0f / lsum;
    uint16_t* orow = static_cast<uint16_t*>(p.out) + ((int64_t)(row + cr) * hq + h) * D + qd * 4;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      const u32x2 w = {pack_bf16x2(acc[dt][0] * inv, acc[dt][1] * inv),
                       pack_bf16x2(acc[dt][2] * inv, acc[dt][3] * inv)};
      *reinterpret_cast<u32x2*>(orow + dt * 16) = w;
    }
  } else {
    const int64_t slot = part_slot(pbase, nparts, nrows * G, g, c, slot_part);
    float* po = p.part_o + slot * D + qd * 4;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) *reinterpret_cast<f32x4*>(po + dt * 16) = acc[dt];
    if (qd == 0) {
      p.part_ml[slot * 2 + 0] = m;
      p.part_ml[slot * 2 + 1] = lsum;
    }
  }
}

hipError_t launch_decode_bf16(const AttnParams& p, hipStream_t stream) {
  const int64_t grid = p.decode_wgs;  // bound on the planner's (task, kv head) pairs
  if (grid <= 0) return hipSuccess;
  if (p.head_dim == 128) {
    hipLaunchKernelGGL(decode_bf16_kernel<128>, dim3((unsigned)grid), dim3(64), 0, stream, p);
  } else {
    hipLaunchKernelGGL(decode_bf16_kernel<64>, dim3((unsigned)grid), dim3(64), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace pa
