// Varlen causal prefill on bf16 MFMA (gfx950): the chunks of a mixed step.
//
// Long prompts run in chunks, so a chunk's rows attend to the prompt's cached context
// plus the chunk's own earlier rows (restatement of "Inside vLLM", section 二, item 1;
// shengyayun.com blog, MVP steps, long-prefill threshold). Prefill is the compute-bound
// side of the step (restatement section 一, scheduler) and the only dense contraction
// of the path, so it runs on the matrix cores.
//
// Work unit: one workgroup = (chunk sequence, tile of R rows, kv head). The query
// "columns" of a kv head are (row, head-in-group) pairs; a strip is 32 of them
// (32 / G rows x G heads, one MFMA N-tile). Each of the NW waves owns NS strips, so
// R = NW * NS * (32 / G) rows. The K/V tiles of the kv head are staged once in LDS and
// shared by every strip of the workgroup.
//
// Keys are staged 64 at a time (4 blocks, gathered through the block table; 128 with
// 8-wave workgroups) and computed in tiles of 64. Per compute tile:
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: A = 32 keys x 16 dims read from LDS,
//    B = Q^T held in registers for the whole tile loop;
//  * the key rows are fed to the MFMA in a fixed permuted order, chosen so that the
//    accumulator elements a lane holds are 8 consecutive keys of one block: they are
//    then directly the B operand of O^T = V^T P^T, and the matching A operand is one
//    16-byte read of the dim-major value tile (8 consecutive tokens of one dimension);
//  * online softmax in the log2 domain with a lazily raised running max: the output is
//    rescaled only when some column's max grows by more than 2^8, which after the first
//    tiles is rare. Exact either way: the same max is used for the weights and the sum;
//  * masked keys (causal, or past the sequence end) are removed by select, and value
//    entries past the sequence end are zeroed while staging, so NaN in unwritten slots
//    cannot leak.
// Staged tiles go from global memory straight into LDS (buffer loads with an LDS
// destination, 16 bytes per lane), double-buffered: the loads of stage s+1 are in flight
// while stage s is multiplied, and one barrier per stage separates the buffers (two
// 32 KB buffers for D = 128).
// Each lane picks the global 16 bytes that belong in its LDS slot, so the tiles land
// XOR-swizzled in 16-byte units and the 16-byte operand reads of a half-wave hit
// distinct banks. The compiler does not count these loads as LDS writes, so the kernel
// waits for them explicitly (vmcnt) before the barrier that publishes a stage.
// Buffer loads rather than global_load_lds: the compiler treats the latter as a flat
// access that may touch LDS, and while one is outstanding (all stage long, by design)
// it drains every LDS read before its first use (lgkmcnt(0)). With buffer loads the
// operand reads of a product are waited for one by one, a few slices ahead of the MFMAs
// that use them.
//
// Workgroups take tasks last-first: last sequence, last rows first, kv head fastest.
// For chunks listed in ascending-context order that starts the longest tiles first.
#include <algorithm>

#include "pa_internal.h"

namespace pa {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazyRescale = 8.0f;  // log2 of the largest weight let through unscaled
constexpr int kTK = 64;              // keys per compute tile
// s_waitcnt immediate for gfx9: vmcnt = 0, expcnt and lgkmcnt left at their maxima.
constexpr int kWaitVmcnt0 = 0x0F70;

__device__ inline bf16x8 as_bf16x8(u32x4 w) { return __builtin_bit_cast(bf16x8, w); }

// max(x[l], x[l ^ 32]) in every lane: v_permlane32_swap exchanges the upper half of its
// first operand with the lower half of its second, so with x in both, each lane ends up
// holding its own value in one result and its partner's in the other.
__device__ inline float max_across_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Key row (within a 32-key half tile) that MFMA row m reads; see the header comment.
__device__ inline int perm_key(int m) {
  return ((m >> 4) << 4) | (((m >> 2) & 1) << 3) | (((m >> 3) & 1) << 2) | (m & 3);
}

// One 16-byte global -> LDS copy per lane (lane i lands at lds_base + 16 i), as a buffer
// load whose resource is one (block, kv head) tile: base is that tile's address (uniform),
// voff the lane's byte offset inside it. The resource's last word (0x00020000) selects a
// 32-bit data format, the usual setting for raw (untyped) buffer loads on this family;
// with stride 0 and num_records = the tile's bytes, an offset past the tile would read
// zeros instead of memory outside it (the offsets here all lie inside).
__device__ __attribute__((always_inline)) inline void lds_dma16(const void* tile, int tile_bytes, int voff,
                                                                uint16_t* lds_base) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(tile), (short)0, tile_bytes,
                                                                     0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base, 16, voff, 0, 0, 0);
}

// 16-byte-unit swizzles of the LDS tiles.
template <int D>
__device__ inline int key_swz(int row) {
  return (row / (128 / D)) & (D / 8 - 1);
}
__device__ inline int val_swz(int dim) { return (dim >> 3) & 1; }

}  // namespace

template <int D, int NW, int NS, bool kPrefix>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void prefill_bf16_kernel(AttnParams p) {
  constexpr int CPR = D / 8;                      // 16-byte chunks per key row
  constexpr int NT = NW * 64;
  // Keys per staged LDS tile: one compute tile, so that two workgroups fit a CU's LDS
  // (with 8-wave workgroups, one per CU, chunks stage two compute tiles per barrier).
  constexpr int kST = (kPrefix || NW < 8) ? kTK : 2 * kTK;
  static_assert((2 * kST * D / 8 / 64) % NW == 0, "tile must split evenly over the waves");
  __shared__ __attribute__((aligned(16))) uint16_t lds[2][2 * kST * D];  // keys, then values

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar addressing
  const int lane = tid & 63;
  const int col = lane & 31;  // MFMA column within a strip
  const int h2 = lane >> 5;   // lane half
  const int G = p.group;
  const int hkv = p.num_kv_heads;
  const int hq = p.num_q_heads;
  const int RW = 32 / G;      // query rows (chunk mode) or decode sequences (prefix mode) per strip
  const int R = NW * NS * RW;
  const int64_t u = blockIdx.x;

  // ---- the task: which keys, which block table, which query columns ----
  // Chunk mode: (chunk sequence, tile of R rows, kv head); rows attend causally to keys
  //   [0, ctx + row]. Prefix mode: (shared-prefix partition, tile of R decode sequences,
  //   kv head); every decode row sees every key of the shared prefix, and the result is
  //   a partial (o, m, l) for the merge kernel.
  int g, kbeg, kmax, L, seq_or_pp;
  const int32_t* __restrict__ bt;
  int q0 = 0, n = 0, ctx = 0, r0 = 0, ct = 0, nds = 0;
  if constexpr (kPrefix) {
    const int pkeys = p.plan_hdr[kHdrPrefixKeys];
    if (pkeys == 0) return;
    nds = p.plan_hdr[kHdrDecSeqs];
    const int n_ct = (nds + R - 1) / R;
    if (u >= (int64_t)p.plan_hdr[kHdrPrefixParts] * n_ct * hkv) return;
    g = (int)(u % hkv);
    const int rest = (int)(u / hkv);
    ct = rest % n_ct;
    const int pp = rest / n_ct;
    const int pplen = p.plan_hdr[kHdrPrefixPartTokens];
    kbeg = pp * pplen;
    kmax = min(pkeys, kbeg + pplen);
    L = pkeys;  // keys at or past the shared prefix are masked (they are not shared)
    seq_or_pp = pp;
    bt = p.block_tables + (int64_t)p.dec_seqs[0] * p.max_blocks;
  } else {
    const int S = p.num_seqs;
    const int total_tiles = p.tile_offsets[S];
    if (u >= (int64_t)total_tiles * hkv) return;
    g = (int)(u % hkv);
    const int tile = total_tiles - 1 - (int)(u / hkv);
    const int i = upper_index(p.tile_offsets, S, tile);
    const int rt = tile - p.tile_offsets[i];
    q0 = p.qsl[i];
    n = p.qsl[i + 1] - q0;
    ctx = p.ctx[i];
    L = p.seq_lens[i];
    r0 = rt * R;
    kbeg = 0;
    kmax = ctx + min(r0 + R, n);  // keys [0, kmax) are seen by some row of the tile
    seq_or_pp = i;
    bt = p.block_tables + (int64_t)i * p.max_blocks;
  }
  const uint16_t* __restrict__ kc = static_cast<const uint16_t*>(p.k_cache);
  const uint16_t* __restrict__ vc = static_cast<const uint16_t*>(p.v_cache);
  const uint16_t* __restrict__ qg = static_cast<const uint16_t*>(p.q);
  uint16_t* __restrict__ og = static_cast<uint16_t*>(p.out);
  // A negative scale is folded into the (exactly negated) queries.
  const uint32_t qsign = p.scale < 0.f ? 0x80008000u : 0u;
  // (floored at a tiny positive value so that masked -inf scores still map to weight 0)
  const float sl2 = fmaxf(fabsf(p.scale) * kLog2e, 1e-30f);

  // ---- per strip: columns, validity, query operands ----
  // srow0: first row (chunk) or first decode-sequence index (prefix) of the strip;
  // crow: this column's row / decode-sequence index; cpos: last key the column sees.
  int srow0[NS], skmax[NS], cpos[NS], crow[NS], qrow[NS];
  // prefix mode: the column's partial slot, looked up before the tile loop so that the
  // dependent loads behind it (decode row, its length, its partial base) overlap the tiles
  int64_t pslot[NS];
  bool cvalid[NS];
  bf16x8 qf[NS][D / 16];
  const int head = g * G + (col % G);
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    if constexpr (kPrefix) {
      srow0[s] = ct * R + (wave * NS + s) * RW;
      crow[s] = srow0[s] + col / G;
      cvalid[s] = (col < RW * G) && (crow[s] < nds);
      skmax[s] = srow0[s] < nds ? kmax : 0;
      cpos[s] = L - 1;
      const int i = p.dec_seqs[cvalid[s] ? crow[s] : 0];
      qrow[s] = p.qsl[i];
      const int nparts = p.plan_hdr[kHdrPrefixParts] + split_parts(p.seq_lens[i] - L, p.plan_hdr[kHdrPartTokens]).n;
      pslot[s] = part_slot(p.part_base[i], nparts, G, g, col % G, seq_or_pp);
    } else {
      srow0[s] = r0 + (wave * NS + s) * RW;
      const int srows = max(0, min(RW, n - srow0[s]));
      skmax[s] = srows > 0 ? ctx + srow0[s] + srows : 0;
      crow[s] = srow0[s] + col / G;
      cvalid[s] = (col < RW * G) && (crow[s] < n);
      // Idle columns mirror the strip's first row so their arithmetic stays finite.
      cpos[s] = cvalid[s] ? ctx + crow[s] : ctx + srow0[s];
      qrow[s] = q0 + (cvalid[s] ? crow[s] : min(srow0[s], n - 1));
    }
    const uint16_t* qr = qg + ((int64_t)qrow[s] * hq + head) * D + h2 * 8;
#pragma unroll
    for (int kq = 0; kq < D / 16; ++kq) {
      u32x4 w = *reinterpret_cast<const u32x4*>(qr + kq * 16);
      w ^= qsign;
      qf[s][kq] = cvalid[s] ? as_bf16x8(w) : bf16x8{};
    }
  }

  f32x16 o[NS][D / 32];
  float m[NS], l[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    m[s] = -INFINITY;
    l[s] = 0.f;
#pragma unroll
    for (int md = 0; md < D / 32; ++md) o[s][md] = f32x16{};
  }

  // ---- staging: key and value tile of keys [kt, kt + kST), global -> LDS directly ----
  // The tile is 32*D 16-byte slots: key slots [0, 16D) then value slots [16D, 32D). Each
  // wave instruction fills 64 consecutive slots (lane i -> slot base + i), so each lane
  // fetches the global 16 bytes that belong in its slot under the XOR swizzle. All 64
  // slots of one instruction lie in one block, so the block id is loaded once per wave.
  // Blocks at or past the sequence end are read from the sequence's first block instead
  // (any valid memory): their keys are masked and their values zeroed before use.
  constexpr int kKeySlots = kST * D / 8;  // 16-byte slots of the key part
  constexpr int kStBlocks = kST / kBlock;
  // Block ids of a staged tile: lane l holds the id of the tile's block l (l < 8); loaded
  // one tile ahead so that the barrier's wait covers them.
  auto load_ids = [&](int kt) {
    const int b = (kt >> 4) + (lane & (kStBlocks - 1));
    return (b * kBlock < L) ? bt[b] : bt[0];
  };
  // Each wave issues kInstK key copies, then as many value copies.
  constexpr int kInstK = kKeySlots / 64 / NW;
  static_assert((kKeySlots / 64) % NW == 0, "key tile must split evenly over the waves");
  auto dma = [&](int buf, int ids) {
#pragma unroll
    for (int j = 0; j < kInstK; ++j) {
      const int gi = wave * kInstK + j;
      const int s = gi * 64 + lane;
      const int row = s / CPR;
      const int gc = (s % CPR) ^ key_swz<D>(row);
      const int64_t phys = __builtin_amdgcn_readlane(ids, (gi * 64 / CPR) >> 4);
      lds_dma16(kc + (phys * hkv + g) * kBlock * D, kBlock * D * 2, ((row & 15) * D + gc * 8) * 2,
                &lds[buf][gi * 64 * 8]);
    }
#pragma unroll
    for (int j = 0; j < kInstK; ++j) {
      const int gi = wave * kInstK + j;
      const int sv = gi * 64 + lane;
      const int dim = (sv >> 1) % D;
      const int gh = (sv & 1) ^ val_swz(dim);
      const int64_t phys = __builtin_amdgcn_readlane(ids, gi * 64 / (2 * D));
      lds_dma16(vc + (phys * hkv + g) * D * kBlock, kBlock * D * 2, (dim * kBlock + gh * 8) * 2,
                &lds[buf][kST * D + gi * 64 * 8]);
    }
  };
  // Zero the value entries of keys [L, kt + kST) in a staged tile (only the tile that
  // holds the sequence end needs it).
  auto zero_tail = [&](int kt, int buf) {
    const int k0 = max(L, kt);
    const int nk = kt + kST - k0;
    for (int x = tid; x < nk * D; x += NT) {
      const int key = k0 - kt + x / D;
      const int dim = x % D;
      const int bl = key >> 4, o = key & 15;
      lds[buf][kST * D + (bl * D + dim) * kBlock + (((o >> 3) ^ val_swz(dim)) * 8) + (o & 7)] = 0;
    }
  };

  // ---- S^T = K Q^T for the 64 keys of one half of a staged key tile ----
  auto qk = [&](int buf, int half, f32x16 (&sc)[NS][2]) {
#pragma unroll
    for (int s = 0; s < NS; ++s) sc[s][0] = sc[s][1] = f32x16{};
    const int row0 = half * kTK + perm_key(col);
    const uint16_t* kr0 = &lds[buf][row0 * D];
    const uint16_t* kr1 = &lds[buf][(32 + row0) * D];
    const int sw0 = key_swz<D>(row0), sw1 = key_swz<D>(32 + row0);
    bf16x8 a0[D / 16], a1[D / 16];
#pragma unroll
    for (int kq = 0; kq < D / 16; ++kq) {
      a0[kq] = *reinterpret_cast<const bf16x8*>(kr0 + (((kq * 2 + h2) ^ sw0) * 8));
      a1[kq] = *reinterpret_cast<const bf16x8*>(kr1 + (((kq * 2 + h2) ^ sw1) * 8));
    }
#pragma unroll
    for (int kq = 0; kq < D / 16; ++kq) {
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        sc[s][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0[kq], qf[s][kq], sc[s][0], 0, 0, 0);
        sc[s][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1[kq], qf[s][kq], sc[s][1], 0, 0, 0);
      }
    }
  };

  // ---- online softmax of one tile's scores (log2 domain, lazy rescale) -> P^T ----
  //   softmax_weights: mask (if asked), running max, weights, packed P^T, partial sums;
  //   softmax_commit:  the rare rescale of the output, then the running sum.
  // The weights of a 16-key block feed that block's PV MFMAs, so the compiler overlaps
  // the exponentials of later blocks with the MFMAs of earlier ones.
  auto softmax_weights = [&](int kt, bool masked, f32x16 (&sc)[NS][2], bf16x8 (&pf)[NS][4], float (&mnew)[NS],
                             float (&psum)[NS], bool& any_raise) {
    any_raise = false;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      // element r of sc[s][mt] is key kt + mt*32 + 16*(r>>3) + 8*h2 + (r&7)
      if (masked) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kt + mt * 32 + 16 * (r >> 3) + 8 * h2 + (r & 7);
            sc[s][mt][r] = key > cpos[s] ? -INFINITY : sc[s][mt][r];
          }
      }
      float mx = sc[s][0][0];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[s][mt][r]);
      mx = max_across_halves(mx);
      const float mxs = mx * sl2;
      const bool raise = mxs > m[s] + kLazyRescale;
      any_raise |= raise;
      mnew[s] = raise ? mxs : m[s];
      const float nm = -mnew[s];
      float ps[4];
#pragma unroll
      for (int ub = 0; ub < 4; ++ub) {
        float pe[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pe[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[s][ub >> 1][(ub & 1) * 8 + e], sl2, nm));
          ps[e & 3] = (ub == 0 && e < 4) ? pe[e] : ps[e & 3] + pe[e];  // no + 0 to start
        }
        const u32x4 w = {pack_bf16x2(pe[0], pe[1]), pack_bf16x2(pe[2], pe[3]),
                         pack_bf16x2(pe[4], pe[5]), pack_bf16x2(pe[6], pe[7])};
        pf[s][ub] = as_bf16x8(w);
      }
      psum[s] = (ps[0] + ps[1]) + (ps[2] + ps[3]);
    }
  };
  auto softmax_commit = [&](const float (&mnew)[NS], const float (&psum)[NS], bool any_raise) {
    if (__builtin_amdgcn_ballot_w64(any_raise)) {
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const float alpha = __builtin_amdgcn_exp2f(m[s] - mnew[s]);
        l[s] *= alpha;
#pragma unroll
        for (int md = 0; md < D / 32; ++md) o[s][md] *= alpha;
      }
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      m[s] = mnew[s];
      l[s] += psum[s];
    }
  };

  // ---- O^T += V^T P^T for one half of a staged value tile ----
  auto pv_load = [&](int buf, int half, bf16x8 (&va)[D / 32][4]) {
#pragma unroll
    for (int ub = 0; ub < 4; ++ub) {
#pragma unroll
      for (int md = 0; md < D / 32; ++md) {
        const int dim = md * 32 + col;
        const int sw = val_swz(dim);
        va[md][ub] = *reinterpret_cast<const bf16x8*>(&lds[buf][kST * D + ((half * 4 + ub) * D + dim) * kBlock + ((h2 ^ sw) * 8)]);
      }
    }
  };
  auto pv = [&](const bf16x8 (&va)[D / 32][4], bf16x8 (&pf)[NS][4]) {
#pragma unroll
    for (int ub = 0; ub < 4; ++ub)
#pragma unroll
      for (int md = 0; md < D / 32; ++md)
#pragma unroll
        for (int s = 0; s < NS; ++s) o[s][md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[md][ub], pf[s][ub], o[s][md], 0, 0, 0);
  };

  // ---- tile loop ----
  // The loads of stage s+1 are in flight while the two compute tiles of stage s are
  // multiplied; the two LDS buffers alternate and one barrier per stage separates them.
  // Waves whose rows need no more keys skip the arithmetic but keep staging and meeting
  // the barrier.
  int wkmax = 0;  // keys this wave's strips need
  int wtm = 1 << 30;  // first tile that needs the mask
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    wkmax = max(wkmax, skmax[s]);
    // tile t holds keys up to 64t + 63; the strip's earliest column sees keys up to
    // ctx + srow0 (chunk) or the whole prefix (prefix)
    wtm = min(wtm, ((kPrefix ? L - 1 : ctx + srow0[s]) + 1) / kTK);
  }

  dma(0, load_ids(kbeg));
  int ids_next = kbeg + kST < kmax ? load_ids(kbeg + kST) : 0;
  int buf = 0;
  for (int kt = kbeg; kt < kmax; kt += kST, buf ^= 1) {
    // The compiler does not count LDS-DMA loads as LDS writes, so the barrier alone
    // would not wait for them: wait for every outstanding vector-memory operation of
    // this wave (this tile's DMA and the next tile's block ids), then publish.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    if (kt + kST > L) {
      zero_tail(kt, buf);
      __syncthreads();
    }
    if (kt + kST < kmax) {  // the other buffer was released by the barrier above
      dma(buf ^ 1, ids_next);
      if (kt + 2 * kST < kmax) ids_next = load_ids(kt + 2 * kST);
    }
#pragma unroll
    for (int half = 0; half < kST / kTK; ++half) {
      const int kh = kt + half * kTK;
      if (kh >= wkmax) break;
      f32x16 sc[NS][2];
      bf16x8 pf[NS][4];
      float mnew[NS], psum[NS];
      bool any_raise;
      bf16x8 va[D / 32][4];
      qk(buf, half, sc);
      pv_load(buf, half, va);
      // Instruction order: the first 3 key slices (6 reads), then each pair of QK MFMAs
      // followed by the reads 3 slices ahead; the value reads fill in behind the last
      // MFMAs and land while the softmax runs.
      __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
      for (int j = 0; j < D / 16 - 3; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * NS, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * NS, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * NS, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * NS, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, D / 8 - 8, 0);
      softmax_weights(kh, kh / kTK >= wtm, sc, pf, mnew, psum, any_raise);
      softmax_commit(mnew, psum, any_raise);
      pv(va, pf);
    }
  }

  // ---- epilogue ----
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const float lt = l[s] + __shfl_xor(l[s], 32);
    if (!cvalid[s]) continue;
    if constexpr (kPrefix) {
      // partial of shared-prefix partition seq_or_pp for decode sequence dec_seqs[crow]:
      // unnormalised o, running max and weight sum (the merge kernel finishes the row)
      const int64_t slot = pslot[s];
      float* po = p.part_o + slot * D + 4 * h2;
#pragma unroll
      for (int md = 0; md < D / 32; ++md)
#pragma unroll
        for (int grp = 0; grp < 4; ++grp)
          *reinterpret_cast<f32x4*>(po + md * 32 + grp * 8) =
              f32x4{o[s][md][grp * 4 + 0], o[s][md][grp * 4 + 1], o[s][md][grp * 4 + 2], o[s][md][grp * 4 + 3]};
      if (h2 == 0) {
        p.part_ml[slot * 2 + 0] = m[s];
        p.part_ml[slot * 2 + 1] = lt;
      }
      continue;
    }
    // normalise, round to bf16, write this lane's 4 x 4 dims per 32
    const float inv = 1.0f / lt;
    uint16_t* orow = og + ((int64_t)qrow[s] * hq + head) * D + 4 * h2;
#pragma unroll
    for (int md = 0; md < D / 32; ++md) {
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        const u32x2 w = {pack_bf16x2(o[s][md][grp * 4 + 0] * inv, o[s][md][grp * 4 + 1] * inv),
                         pack_bf16x2(o[s][md][grp * 4 + 2] * inv, o[s][md][grp * 4 + 3] * inv)};
        *reinterpret_cast<u32x2*>(orow + md * 32 + grp * 8) = w;
      }
    }
  }
}

// Workgroup shape: waves per workgroup and 32-column strips per wave. Two 4-wave
// workgroups share a CU (one wave of each per SIMD, 64 KB of LDS each); each meets only
// its own barriers, so the two waves of a SIMD drift out of step and one's MFMA work
// overlaps the other's softmax. One 8-wave workgroup per CU keeps them in lockstep:
// 2.5% slower, although it stages each key/value tile for twice the rows.
constexpr int kPrefillWaves = 4;
constexpr int kPrefillStrips = 1;

int prefill_rows_per_tile(int group) { return kPrefillWaves * kPrefillStrips * (32 / group); }

hipError_t launch_prefill_bf16(const AttnParams& p, hipStream_t stream) {
  if (p.num_seqs == 0 || p.num_tokens < 2) return hipSuccess;
  const int R = prefill_rows_per_tile(p.group);
  // Upper bound on the tiles the planner can emit: every chunk has >= 2 rows.
  const int64_t chunks = std::min<int64_t>(p.num_seqs, p.num_tokens / 2);
  const int64_t tiles = (p.num_tokens + (int64_t)(R - 1) * chunks) / R + 1;
  const int64_t grid = tiles * p.num_kv_heads;
  if (p.head_dim == 128) {
    hipLaunchKernelGGL((prefill_bf16_kernel<128, kPrefillWaves, kPrefillStrips, false>), dim3((unsigned)grid),
                       dim3(kPrefillWaves * 64), 0, stream, p);
  } else {
    hipLaunchKernelGGL((prefill_bf16_kernel<64, kPrefillWaves, kPrefillStrips, false>), dim3((unsigned)grid),
                       dim3(kPrefillWaves * 64), 0, stream, p);
  }
  return hipGetLastError();
}

hipError_t launch_prefix_bf16(const AttnParams& p, hipStream_t stream) {
  if (p.num_seqs < 2) return hipSuccess;
  // Upper bound on the planner's shared-prefix tasks, pparts * ceil(rows / R) with
  // pparts * rows <= max(kPrefixSlotRows, rows) and rows <= S:
  //   pparts * ceil(rows / R) <= (pparts * rows + pparts * (R - 1)) / R,
  // pparts at most the prefix (shorter than the longest sequence) over the shortest
  // partition, and at most kPrefixSlotRows / 2 (there are at least two decode rows).
  // Workgroups past the planned tasks exit at once.
  const int64_t R = prefill_rows_per_tile(p.group);
  const int64_t max_len = (int64_t)p.max_blocks * kBlock;
  // shortest prefix partition: min(P, 512) in whole 64-key tiles, P >= kMinPartTokens
  // unless the caller fixed it
  const int64_t pmin = (std::min(p.part_tokens ? p.part_tokens : kMinPartTokens, 512) + 63) / 64 * 64;
  const int64_t pparts = std::min<int64_t>((max_len + pmin - 1) / pmin, kPrefixSlotRows / 2);
  const int64_t rows = std::min<int64_t>(p.num_seqs, p.num_tokens);
  const int64_t tiles = (std::max<int64_t>(kPrefixSlotRows, rows) + pparts * (R - 1) + R - 1) / R;
  const int64_t grid = tiles * p.num_kv_heads;
  if (p.head_dim == 128) {
    hipLaunchKernelGGL((prefill_bf16_kernel<128, kPrefillWaves, kPrefillStrips, true>), dim3((unsigned)grid),
                       dim3(kPrefillWaves * 64), 0, stream, p);
  } else {
    hipLaunchKernelGGL((prefill_bf16_kernel<64, kPrefillWaves, kPrefillStrips, true>), dim3((unsigned)grid),
                       dim3(kPrefillWaves * 64), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace pa
