// Split-KV decode attention for grouped-query heads, VALU path (gfx950).
//
// Computes, for each (batch b, KV head g, group of GH query heads, KV split),
// the partial triple over the split's tokens (aclnnRingAttentionUpdate,
// "功能说明": attn_out, softmax_max, softmax_sum) of
//   Softmax(scale * q K^T) V          (aclnnIncreFlashAttentionV3, "Function")
// where the KV rows are read through the block table of the page attention
// scenario (aclnnIncreFlashAttentionV3, "Constraints": layout
// (blocknum, KV_N, blocksize, D)) or from a padded contiguous (B, N, S, D)
// buffer, and int8 K/V are dequantised per channel in registers
// (antiquantScale / antiquantOffset, "Parameters").
//
// Work decomposition.  One workgroup = 4 waves = one (b, g, head group,
// split); workgroups are dispatched longest sequence first.  The waves take
// the split's steps round robin.  Inside a wave, C = D/16 lanes share one
// token row (16 channels per lane, loaded as 16-byte chunks so that each load
// instruction reads whole 128-byte row segments), so a step covers 64/C
// tokens.  Each wave streams its steps through a private LDS ring filled by
// direct HBM -> LDS loads issued STAGES-1 steps ahead.  q for the GH heads
// stays in registers.  Per step: QK^T (packed dot2 for f16/bf16, fp32 FMA
// for f32 and int8), a C-lane DPP reduction, a lazy softmax rescale per lane
// group (the running reference moves only when a score exceeds it by 2^8),
// then P V in fp32 FMAs.  At the end the waves merge their (max, sum, acc)
// through LDS and the workgroup writes the normalised partial.
#include "common.hpp"
#include "kernels.hpp"

namespace ifa {
namespace {

template <int KV>
struct KvInfo;
template <>
struct KvInfo<kF32> { static constexpr int esz = 4; };
template <>
struct KvInfo<kF16> { static constexpr int esz = 2; };
template <>
struct KvInfo<kBF16> { static constexpr int esz = 2; };
template <>
struct KvInfo<kI8> { static constexpr int esz = 1; };

// Element e (0..15) of a lane's 16 channels, as fp32.  Chunk i = e / E holds
// E = 16 / esz consecutive channels.  int8 values arrive biased by +128
// (bytes xor 0x80) and are converted as unsigned bytes.
template <int KV>
__device__ __forceinline__ float elem_f32(const u32x4 (&r)[KvInfo<KV>::esz], int e) {
  constexpr int E = 16 / KvInfo<KV>::esz;
  const int i = e / E, k = e % E;
  if constexpr (KV == kF32) {
    return __uint_as_float(word(r[i], k));
  } else if constexpr (KV == kBF16) {
    const uint32_t w = word(r[i], k >> 1);
    return (k & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
  } else if constexpr (KV == kF16) {
    const uint32_t w = word(r[i], k >> 1);
    half2_t h = __builtin_bit_cast(half2_t, w);
    return (k & 1) ? (float)h[1] : (float)h[0];
  } else {
    // (float)(byte) of the biased word maps to v_cvt_f32_ubyte{0..3}
    const uint32_t w = word(r[0], k >> 2) ^ 0x80808080u;
    return (float)((w >> (8 * (k & 3))) & 0xffu);
  }
}

// Direct HBM -> LDS load of 16 bytes per lane (gfx950
// global_load_lds_dwordx4): lane l reads base + voff and its 16 bytes land at
// LDS byte address lds + 16 * l.  `base` and `lds` are wave-uniform.
//
// Issued from inline asm on purpose: the compiler then neither tracks these
// loads nor guards LDS reads against them (it would wait for every
// outstanding load before each LDS read), and the kernel orders the ring with
// explicit vmcnt waits instead (wait_vmem).  No other vector-memory operation
// is issued inside the streaming loop, so the counts are exact.
__device__ __forceinline__ void dma16(const char* base, uint32_t voff, uint32_t lds) {
#if IFA_GQA_NT_LOADS
  // streaming hint: KV rows are read once
  asm volatile("global_load_lds_dwordx4 %0, %1 offset:0 nt" ::"v"(voff), "s"(base), "{m0}"(lds) : "memory");
#else
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "{m0}"(lds) : "memory");
#endif
}

// Wait until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vmem() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Wait for this wave's LDS reads (and scalar loads) to complete.
__device__ __forceinline__ void wait_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// Wait until at most n * LOADS vector-memory operations are in flight, for a
// run-time n in [0, NMAX] (the count is an immediate of s_waitcnt).
template <int NMAX, int LOADS>
__device__ __forceinline__ void wait_vmem_steps(int n) {
  if constexpr (NMAX <= 0) {
    wait_vmem<0>();
  } else {
    if (n >= NMAX) wait_vmem<NMAX * LOADS>();
    else wait_vmem_steps<NMAX - 1, LOADS>(n);
  }
}

// Make the compiler complete the loads behind `x` here: an empty asm that
// reads the register forces the wait before this point instead of at the
// first use inside the streaming loop, where it would also drain the ring.
template <typename T>
__device__ __forceinline__ void settle(const T& x) {
  asm volatile("" ::"v"(x));
}

// LDS byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

#ifndef IFA_GQA_NT_LOADS
#define IFA_GQA_NT_LOADS 1
#endif
// Bytes of the per-wave LDS ring that K/V steps stream through: two 4-KB
// steps for 16-bit K/V (measured on the paged bf16 decode, about 1 us faster
// than three); six 2-KB steps for int8, whose loop takes steps in pairs.
#ifndef IFA_GQA_RING_BYTES
#define IFA_GQA_RING_BYTES 8192
#endif
constexpr int kRingBytesPerWave = IFA_GQA_RING_BYTES;
constexpr int kRingBytesPerWaveI8 = 12288;

// The value that lane ^ X holds, X in {4, 8, 16, 32}.  The permlane swaps,
// given one register twice, return it with the partner row's half swapped in
// (first result: own lanes where the lane bit is clear), so the partner's
// value is the first result in the upper half and the second in the lower.
template <int X>
__device__ __forceinline__ float xor_lane(float x) {
  static_assert(X == 4 || X == 8 || X == 16 || X == 32, "lane distance");
  if constexpr (X == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
  } else if constexpr (X == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float((threadIdx.x & 16) ? r[0] : r[1]);
  } else if constexpr (X == 8) {
    return dpp_f32<kDppRowRor8>(x);  // rotation by 8 inside a row of 16 = lane ^ 8
  } else {
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), (4 << 10) | 0x1f));  // lane ^ 4
  }
}

// One halving step of a reduce-scatter over lanes l and l ^ X: the lane with
// bit X set keeps the upper half of v[0, 2H), the other the lower half, each
// adding the partner's copy of the half it keeps.
template <int H, int X>
__device__ __forceinline__ void reduce_scatter_step(float (&v)[16]) {
  const bool upper = (threadIdx.x & X) != 0;
#pragma unroll
  for (int i = 0; i < H; ++i) {
    const float lo = v[i], hi = v[i + H];
    const float send = upper ? lo : hi;
    v[i] = (upper ? hi : lo) + xor_lane<X>(send);
  }
}

template <int QT, int KV, int D, int GH>
struct GqaShape {
  static constexpr int C = D / 16;           // lanes per token row
  static constexpr int TOK = 64 / C;         // tokens per step
  static constexpr int ESZ = KvInfo<KV>::esz;
  static constexpr int E = 16 / ESZ;         // channels per 16-byte chunk
  static constexpr int NCH = ESZ;            // chunks per lane per row
  static constexpr int ROWB = D * ESZ;       // bytes per token row
  static constexpr int STEP_BYTES = 2 * NCH * 1024;  // K and V of one step, whole wave
  // eight heads per workgroup leave one wave per SIMD (registers), so that
  // instantiation gets a deeper ring to keep enough loads in flight
  static constexpr int RING_WAVE = GH == 8 ? 32768 : (KV == kI8 ? kRingBytesPerWaveI8 : kRingBytesPerWave);
  static constexpr int STAGES_FIT = RING_WAVE / STEP_BYTES < 2 ? 2 : RING_WAVE / STEP_BYTES;
  static constexpr int STAGES = (STAGES_FIT - 1) * 2 * NCH > 63 ? 63 / (2 * NCH) + 1 : STAGES_FIT;
  static constexpr int LOADS = 2 * NCH;      // load instructions per step
  static constexpr int RING_BYTES = 4 * STAGES * STEP_BYTES;
  static constexpr int MERGE_BYTES = 4 * GH * D * 4 + 2 * 4 * GH * 4;  // [4][GH][D] sums, [4][GH] max and sum
  static constexpr int SMEM = RING_BYTES > MERGE_BYTES ? RING_BYTES : MERGE_BYTES;
  static_assert(STAGES * STEP_BYTES >= kLongestFirstMaxBatch * 4, "rank keys fit a wave's ring");
};

template <int QT, int KV, int D, int GH, bool PAGED>
__global__ void __launch_bounds__(256) gqa_splitkv_kernel(const GqaLaunch a, int work_items) {
  using S = GqaShape<QT, KV, D, GH>;
  constexpr int C = S::C, TOK = S::TOK, E = S::E, NCH = S::NCH, ROWB = S::ROWB;
  constexpr int STAGES = S::STAGES, LOADS = S::LOADS;
  constexpr bool DOT2 = (KV == kF16 || KV == kBF16);
  // int8 K: q' = q * K scale is kept as packed fp16 pairs and every K byte
  // pair becomes the fp16 pair (1024 + byte ^ 0x80) with one byte permute
  // (exact: 1024 <= value < 2048 has unit spacing), so QK^T runs on packed
  // fp16 dot products like the f16 path
  constexpr bool I8DOT = (KV == kI8);
  constexpr bool PACKQ = DOT2 || I8DOT;
  constexpr float kRescale = 8.f;    // log2 headroom before the running reference moves
  constexpr float kMrefInit = -1e30f;  // finite, so exp2(-inf - mref) is 0, never NaN
  static_assert(D % 16 == 0 && C >= 4 && STAGES >= 2, "shape");

  __shared__ __attribute__((aligned(16))) char smem[S::SMEM];

  // Work items in dispatch order: consecutive workgroups go round robin to
  // the XCDs, so with the longest-first order every XCD receives an equal
  // mix of long and short items.
  // Head groups of one KV head read the same K/V rows.  Workgroups go round
  // robin to the 8 XCDs, so the head groups of an item are placed 8 ids
  // apart: they run on the same XCD at about the same time and the later
  // reads hit its L2 instead of HBM.
  const int HG = a.rows_kv / GH;
  const int span = 8 * HG;
  const int hg = (blockIdx.x % span) / 8;
  int rem = (blockIdx.x / span) * 8 + blockIdx.x % 8;  // item without the head group
  if (rem >= work_items / HG) return;
  const int split = rem % a.n_split; rem /= a.n_split;
  const int g = rem % a.n_kv; rem /= a.n_kv;
  int b = rem, L;
  if (a.plan) {
    // longest-first: the planning kernel ranked the sequences for this launch
    const int64_t pl = ld_uniform(reinterpret_cast<const int64_t*>(a.plan), rem);  // (sequence, length)
    b = (int)(uint32_t)pl;
    L = (int)(pl >> 32);
  } else if (a.longest_first) {
    // longest-first, ranked here by every wave; the keys use this wave's part
    // of the ring, which no load has reached yet
    uint32_t* keys = reinterpret_cast<uint32_t*>(smem + (threadIdx.x >> 6) * (STAGES * S::STEP_BYTES));
    const BatchPick pick = batch_of_rank(rem, a.seq_lens, a.batch, a.s_cap, keys);
    b = pick.b;
    L = pick.len;
  } else {
    const int64_t L64 = a.seq_lens[b];
    L = (int)(L64 < 0 ? 0 : (L64 > a.s_cap ? a.s_cap : L64));
  }
  const int per = (int)split_chunk(L, a.n_split);
  const int start = split * per;
  const int end = min(L, start + per);
  if (start >= end) return;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t = lane / C, c = lane % C;
  // Query row x of this workgroup: row hg * GH + x of the KV head's q_seq *
  // group rows, query token major; its index in (B, q_seq, N_q).  With one
  // query token this is head g * group + hg * GH + x of sequence b.
  auto qrow_of = [&](int x) -> int64_t {
    const int rr = hg * GH + x;
    const int i = rr / a.group;
    return ((int64_t)b * a.q_seq + i) * a.n_q + g * a.group + (rr - i * a.group);
  };
  // Multi-token masks: bit k of vis[x] is set when row x attends to draft
  // token k, the token at position draft0 + k (rows attend to every token
  // before draft0).  Wave-uniform.
  const bool masked = a.mask_mode != 0;
  const int draft0 = L - a.q_seq;
  uint32_t vis[GH];
#pragma unroll
  for (int x = 0; x < GH; ++x) {
    vis[x] = ~0u;
    if (masked) {
      const int i = (hg * GH + x) / a.group;
      if (a.mask_mode == 3) {
        vis[x] = (2u << i) - 1u;  // rightDownCausal: draft tokens k <= i
      } else {
        const int k = threadIdx.x & 63;
        const uint8_t m = k < a.q_seq ? a.tree_mask[((int64_t)b * a.q_seq + i) * a.q_seq + k] : 1;
        vis[x] = (uint32_t)__builtin_amdgcn_ballot_w64(m == 0);
      }
    }
  }
  const int nsteps = (end - start + TOK - 1) / TOK;

  const char* kbase = static_cast<const char*>(a.k);
  const char* vbase = static_cast<const char*>(a.v);
  char* ring = smem + wave * (STAGES * S::STEP_BYTES);  // this wave's stages: [K chunks | V chunks]
  const uint32_t ring_lds = lds_addr(ring);

  // Block-table slice of the split: lane k holds the id of the split's k-th
  // cache block, fetched once through scalar loads (which do not queue behind
  // the CU's ring loads); the loop reads it with v_readlane, so it issues no
  // scalar loads, whose waits would also hold back the LDS reads.  A split
  // spanning more than 64 blocks reads the rest with scalar loads.
  const uint32_t bi0 = PAGED ? fast_div((uint32_t)start, a.bs_magic, a.bs_shift) : 0;
  int tbl = 0;
  if constexpr (PAGED) {
    const int nblk = (int)fast_div((uint32_t)(end - 1), a.bs_magic, a.bs_shift) - (int)bi0 + 1;  // in the row
    tbl = lanes_from_scalar_loads(a.block_table + (int64_t)b * a.max_blocks + bi0, nblk < 64 ? nblk : 64, 0);
  }

  // First cache row of step `st`: TOK tokens that lie inside one block
  // (splits start on 16-token boundaries, the block size is a multiple of 16).
  auto step_row = [&](int st) -> uint32_t {
    const int j0 = start + TOK * st;
    if constexpr (PAGED) {
      const uint32_t bi = fast_div((uint32_t)j0, a.bs_magic, a.bs_shift);
      const uint32_t k = bi - bi0;
      int blk = k < 64 ? __builtin_amdgcn_readlane(tbl, k) : ld_uniform(a.block_table, (int64_t)b * a.max_blocks + bi);
      blk = blk < 0 ? 0 : (blk >= a.num_blocks ? a.num_blocks - 1 : blk);
      const uint32_t slot = (uint32_t)j0 - bi * (uint32_t)a.block_size;
      if (a.token_major)  // (blocks, block_size, N_kv, D)
        return ((uint32_t)blk * (uint32_t)a.block_size + slot) * (uint32_t)a.n_kv + (uint32_t)g;
      return ((uint32_t)blk * (uint32_t)a.n_kv + (uint32_t)g) * (uint32_t)a.block_size + slot;
    } else {
      if (a.token_major)  // (B, s_cap, N_kv, D)
        return ((uint32_t)b * (uint32_t)a.s_cap + (uint32_t)j0) * (uint32_t)a.n_kv + (uint32_t)g;
      return ((uint32_t)b * (uint32_t)a.n_kv + (uint32_t)g) * (uint32_t)a.s_cap + (uint32_t)j0;
    }
  };
  // bytes between consecutive tokens of one KV head
  const uint32_t tok_bytes = a.token_major ? (uint32_t)a.n_kv * ROWB : (uint32_t)ROWB;

  // Queue the direct-to-LDS loads of step `st` (< nsteps) into ring stage
  // `slot`.  Lanes past the split's end read its last valid row: finite data
  // that the softmax weights with exactly 0.
  auto issue = [&](int st, int slot) {
    const uint32_t row0 = step_row(st);
    const int r = min(t, end - 1 - (start + TOK * st));
    const uint32_t off = (uint32_t)r * tok_bytes + 16u * c;
    const char* kb = kbase + (uint64_t)row0 * ROWB;
    const char* vb = vbase + (uint64_t)row0 * ROWB;
    const uint32_t dst = ring_lds + slot * S::STEP_BYTES;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      dma16(kb, off + 16 * C * i, dst + 1024 * i);
      dma16(vb, off + 16 * C * i, dst + 1024 * (NCH + i));
    }
  };

  // running state per lane (over the tokens of its lane group):
  // mref: reference max, mtrue: true max, lsum / acc relative to mref
  float mref[GH], mtrue[GH], lsum[GH], acc[GH][16];
#pragma unroll
  for (int h = 0; h < GH; ++h) {
    mref[h] = kMrefInit;
    mtrue[h] = kNegInf;
    lsum[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[h][e] = 0.f;
  }

  if (wave < nsteps) {
    // prologue: up to STAGES of this wave's steps in flight, one per stage
#pragma unroll
    for (int k = 0; k < STAGES; ++k)
      if (wave + 4 * k < nsteps) issue(wave + 4 * k, k);

    // ---- q (and the int8 K-side constant) for this lane's 16 channels ----
    // channel of element e: E * ((e / E) * C + c) + e % E
    float qf[PACKQ ? 1 : GH][PACKQ ? 1 : 16];
    uint32_t qp[PACKQ ? GH : 1][PACKQ ? 8 : 1];
    float kconst[GH];  // int8: sum_d q'_d (offset_d - 1152), with q' as rounded to fp16
    // q in K's dtype and 16-byte aligned: the lane's 16 channels are two runs
    // of 8 (channels 8c.. and 8(C + c)..), i.e. two 16-byte loads per head
    const bool q16 = DOT2 && (reinterpret_cast<uintptr_t>(a.q) & 15) == 0;
    if (q16) {
#pragma unroll
      for (int h = 0; h < GH; ++h) {
        const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + qrow_of(h) * D;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(qrow + 8 * (c + C * i));
#pragma unroll
          for (int w = 0; w < 4; ++w) qp[h][4 * i + w] = word(v, w);
        }
        kconst[h] = 0.f;
      }
    }
#pragma unroll
    for (int h = 0; h < GH && !q16; ++h) {
      const int64_t qrow = qrow_of(h) * D;
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int d = E * ((e / E) * C + c) + e % E;
        if constexpr (DOT2) {
          // q has the dtype of K here: repack its raw bits into pairs
          const uint32_t bits = static_cast<const uint16_t*>(a.q)[qrow + d];
          if (e & 1) qp[h][e >> 1] |= bits << 16; else qp[h][e >> 1] = bits;
        } else if constexpr (I8DOT) {
          // x_hat = (x + offset) * scale with x = f - 1152, f = 1024 + (x ^ 0x80)
          const int kq = g * a.aq_stride_g + d * a.aq_stride_d;  // K parameters (index 0)
          const _Float16 qh = (_Float16)(load_as_f32<QT>(a.q, qrow + d) * a.aq_scale[kq]);
          part = fmaf((float)qh, a.aq_offset[kq] - 1152.f, part);
          const uint32_t bits = __builtin_bit_cast(uint16_t, qh);
          if (e & 1) qp[h][e >> 1] |= bits << 16; else qp[h][e >> 1] = bits;
        } else {
          float qv = load_as_f32<QT>(a.q, qrow + d);
          if constexpr (KV == kI8) {
            const int kq = g * a.aq_stride_g + d * a.aq_stride_d;
            qv *= a.aq_scale[kq];
            part = fmaf(qv, a.aq_offset[kq] - 128.f, part);
          }
          qf[h][e] = qv;
        }
      }
      kconst[h] = (KV == kI8) ? group_sum<C>(part) : 0.f;
    }
#pragma unroll
    for (int h = 0; h < GH; ++h) {
      settle(kconst[h]);
      if constexpr (PACKQ) {
#pragma unroll
        for (int p = 0; p < 8; ++p) settle(qp[h][p]);
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) settle(qf[h][e]);
      }
    }

    if constexpr (I8DOT) {
      // int8: two of this wave's steps per iteration, the lane's token of
      // each.  V becomes fp16 pairs (1024 + biased byte of step j, of step
      // j+1) per channel, so P V is one v_dot2 per channel and head on the
      // pair of softmax weights rounded to fp16.  The row sum takes the same
      // rounded weights, so the 1024 bias divides out exactly (the epilogue
      // removes 1024 + 128 with the V offset).
      int slot = 0;
      for (int st = wave; st < nsteps; st += 8) {
        const bool two = st + 4 < nsteps;
        // wait for both steps; the loads of this wave's steps queued after
        // the second one (at most STAGES-2 of them: two stages are refilled
        // per iteration) stay in flight
        const int later = (nsteps - 1 - st) / 4 - (two ? 1 : 0);
        wait_vmem_steps<STAGES - 2, LOADS>(later < STAGES - 2 ? later : STAGES - 2);
        const int slot1 = two ? (slot + 1 == STAGES ? 0 : slot + 1) : slot;
        const char* src0 = ring + slot * S::STEP_BYTES + 16 * lane;
        const char* src1 = ring + slot1 * S::STEP_BYTES + 16 * lane;
        const u32x4 kr0 = *reinterpret_cast<const u32x4*>(src0);
        const u32x4 vr0 = *reinterpret_cast<const u32x4*>(src0 + 1024);
        const u32x4 kr1 = *reinterpret_cast<const u32x4*>(src1);
        const u32x4 vr1 = *reinterpret_cast<const u32x4*>(src1 + 1024);
        if (st + 4 * STAGES < nsteps) {
          wait_lds();  // the direct loads below overwrite these stages
          issue(st + 4 * STAGES, slot);
          if (st + 4 + 4 * STAGES < nsteps) issue(st + 4 + 4 * STAGES, slot1);
        }

        const bool valid0 = start + TOK * st + t < end;
        const bool valid1 = two && start + TOK * (st + 4) + t < end;
        uint32_t k0[8], k1[8];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t b0 = word(kr0, w) ^ 0x80808080u, b1 = word(kr1, w) ^ 0x80808080u;
          k0[2 * w] = __builtin_amdgcn_perm(0x64646464u, b0, 0x04010400u);
          k0[2 * w + 1] = __builtin_amdgcn_perm(0x64646464u, b0, 0x04030402u);
          k1[2 * w] = __builtin_amdgcn_perm(0x64646464u, b1, 0x04010400u);
          k1[2 * w + 1] = __builtin_amdgcn_perm(0x64646464u, b1, 0x04030402u);
        }
        float s0[GH], s1[GH];
        bool need = false;
#pragma unroll
        for (int h = 0; h < GH; ++h) {
          float d0 = 0.f, d1 = 0.f;
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            d0 = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, qp[h][q]), __builtin_bit_cast(half2_t, k0[q]), d0,
                                        false);
            d1 = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, qp[h][q]), __builtin_bit_cast(half2_t, k1[q]), d1,
                                        false);
          }
          d0 = group_sum<C>(d0) + kconst[h];
          d1 = group_sum<C>(d1) + kconst[h];
          s0[h] = valid0 ? d0 * a.scale_log2 : kNegInf;
          s1[h] = valid1 ? d1 * a.scale_log2 : kNegInf;
        }
        if (masked && start + TOK * (st + (two ? 5 : 1)) > draft0) {  // the steps reach the draft tokens
          const int k0 = start + TOK * st + t - draft0, k1 = k0 + 4 * TOK;
#pragma unroll
          for (int h = 0; h < GH; ++h) {
            if (k0 >= 0 && k0 < 32 && !((vis[h] >> k0) & 1u)) s0[h] = kNegInf;
            if (k1 >= 0 && k1 < 32 && !((vis[h] >> k1) & 1u)) s1[h] = kNegInf;
          }
        }
#pragma unroll
        for (int h = 0; h < GH; ++h) {
          const float sm = fmaxf(s0[h], s1[h]);
          mtrue[h] = fmaxf(mtrue[h], sm);
          need |= sm > mref[h] + kRescale;
        }
        if (__builtin_amdgcn_ballot_w64(need)) {  // rare after the first steps
#pragma unroll
          for (int h = 0; h < GH; ++h) {
            const float sm = fmaxf(s0[h], s1[h]);
            const float mnew = sm > mref[h] + kRescale ? sm : mref[h];
            const float alpha = fast_exp2(mref[h] - mnew);  // 0 on the first valid token
            lsum[h] *= alpha;
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[h][e] *= alpha;
            mref[h] = mnew;
          }
        }
        // softmax weights of the two tokens as one fp16 pair (<= 2^8; 0 for
        // invalid tokens), and the row sum of exactly those values
        half2_t pw[GH];
        const half2_t ones = {(_Float16)1.f, (_Float16)1.f};
#pragma unroll
        for (int h = 0; h < GH; ++h) {
          pw[h] = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_pkrtz(fast_exp2(s0[h] - mref[h]), fast_exp2(s1[h] - mref[h])));
          lsum[h] = __builtin_amdgcn_fdot2(pw[h], ones, lsum[h], false);
        }
        // channel pairs across the two steps: bytes (e of step j, e of step
        // j+1) interleaved, biased, then widened to (1024 + byte) fp16
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t a0 = word(vr0, w), a1 = word(vr1, w);
          const uint32_t lo = __builtin_amdgcn_perm(a1, a0, 0x05010400u) ^ 0x80808080u;  // e0 j, e0 j+1, e1 j, e1 j+1
          const uint32_t hi = __builtin_amdgcn_perm(a1, a0, 0x07030602u) ^ 0x80808080u;  // e2 .., e3 ..
          const uint32_t vp[4] = {__builtin_amdgcn_perm(0x64646464u, lo, 0x04010400u),
                                  __builtin_amdgcn_perm(0x64646464u, lo, 0x04030402u),
                                  __builtin_amdgcn_perm(0x64646464u, hi, 0x04010400u),
                                  __builtin_amdgcn_perm(0x64646464u, hi, 0x04030402u)};
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int h = 0; h < GH; ++h)
              acc[h][4 * w + q] = __builtin_amdgcn_fdot2(pw[h], __builtin_bit_cast(half2_t, vp[q]), acc[h][4 * w + q], false);
        }
        slot = slot1 + 1 == STAGES ? 0 : slot1 + 1;
      }
    } else {
      int slot = 0;
      for (int st = wave; st < nsteps; st += 4) {
        // wait for step st; the loads of this wave's later steps already queued
        // (at most STAGES-1 of them) stay in flight
        const int later = (nsteps - 1 - st) / 4;
        if (later >= STAGES - 1) wait_vmem<(STAGES - 1) * LOADS>();
        else wait_vmem_steps<STAGES - 2, LOADS>(later);
        // Copy the step out of its stage and queue the step STAGES ahead into
        // it at once: the stage is free again after the LDS reads rather than
        // after the whole step's arithmetic, so the full ring stays in flight.
        const char* src = ring + slot * S::STEP_BYTES + 16 * lane;
        u32x4 kr[NCH], vr[NCH];
  #pragma unroll
        for (int i = 0; i < NCH; ++i) {
          kr[i] = *reinterpret_cast<const u32x4*>(src + 1024 * i);
          vr[i] = *reinterpret_cast<const u32x4*>(src + 1024 * (NCH + i));
        }
        if (st + 4 * STAGES < nsteps) {
          wait_lds();  // the direct loads below overwrite this stage
          issue(st + 4 * STAGES, slot);
        }

        const bool valid = start + TOK * st + t < end;
        uint32_t kf16[I8DOT ? 8 : 1];  // int8 K as fp16 pairs (1024 + biased byte)
        if constexpr (I8DOT) {
  #pragma unroll
          for (int w = 0; w < 4; ++w) {
            const uint32_t bw = word(kr[0], w) ^ 0x80808080u;
            kf16[2 * w] = __builtin_amdgcn_perm(0x64646464u, bw, 0x04010400u);
            kf16[2 * w + 1] = __builtin_amdgcn_perm(0x64646464u, bw, 0x04030402u);
          }
        }
        float s[GH];
        bool need = false;
  #pragma unroll
        for (int h = 0; h < GH; ++h) {
          float part = 0.f;
          if constexpr (KV == kBF16) {
  #pragma unroll
            for (int p = 0; p < 8; ++p)
              part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, qp[h][p]),
                                                     __builtin_bit_cast(bf162_t, word(kr[p / 4], p % 4)), part, false);
          } else if constexpr (KV == kF16) {
  #pragma unroll
            for (int p = 0; p < 8; ++p)
              part = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, qp[h][p]),
                                            __builtin_bit_cast(half2_t, word(kr[p / 4], p % 4)), part, false);
          } else if constexpr (I8DOT) {
  #pragma unroll
            for (int p = 0; p < 8; ++p)
              part = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, qp[h][p]), __builtin_bit_cast(half2_t, kf16[p]),
                                            part, false);
          } else {
  #pragma unroll
            for (int e = 0; e < 16; ++e) part = fmaf(qf[h][e], elem_f32<KV>(kr, e), part);
          }
          float dot = group_sum<C>(part);
          if constexpr (KV == kI8) dot += kconst[h];
          s[h] = valid ? dot * a.scale_log2 : kNegInf;
        }
        if (masked && start + TOK * (st + 1) > draft0) {  // the step reaches the draft tokens
          const int k = start + TOK * st + t - draft0;
#pragma unroll
          for (int h = 0; h < GH; ++h)
            if (k >= 0 && k < 32 && !((vis[h] >> k) & 1u)) s[h] = kNegInf;  // k < q_seq for valid tokens
        }
#pragma unroll
        for (int h = 0; h < GH; ++h) {
          mtrue[h] = fmaxf(mtrue[h], s[h]);
          need |= s[h] > mref[h] + kRescale;
        }
        if (__builtin_amdgcn_ballot_w64(need)) {  // rare after the first step
  #pragma unroll
          for (int h = 0; h < GH; ++h) {
            const float mnew = s[h] > mref[h] + kRescale ? s[h] : mref[h];
            const float alpha = fast_exp2(mref[h] - mnew);  // 0 on the first valid token
            lsum[h] *= alpha;
  #pragma unroll
            for (int e = 0; e < 16; ++e) acc[h][e] *= alpha;
            mref[h] = mnew;
          }
        }
        float p[GH];
  #pragma unroll
        for (int h = 0; h < GH; ++h) {
          p[h] = fast_exp2(s[h] - mref[h]);  // <= 2^8; 0 for invalid lanes
          lsum[h] += p[h];
        }
  #pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float vf = elem_f32<KV>(vr, e);
  #pragma unroll
          for (int h = 0; h < GH; ++h) acc[h][e] = fmaf(p[h], vf, acc[h][e]);
        }
        slot = slot == STAGES - 1 ? 0 : slot + 1;
      }
    }
  }
  // every queued load has been waited for: the ring is free for the merge

  // ---- merge the lane groups of the wave: common max, rescale, sum ----
  float mw[GH];
#pragma unroll
  for (int h = 0; h < GH; ++h) {
    mw[h] = strided_max<C>(mtrue[h]);
    // lanes that saw no valid token hold lsum = acc = 0 and mref = kMrefInit
    const float f = mref[h] == kMrefInit ? 0.f : fast_exp2(mref[h] - mw[h]);
    lsum[h] = strided_sum<C>(lsum[h] * f);
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[h][e] *= f;
    // reduce-scatter over the TOK token lanes (lane = t C + c, so the bits
    // of t are lane bits 5, 4, ... down to log2 C): each step halves the
    // element range by the next lower bit of t, and token lane t ends with
    // the sums of elements EPL t .. EPL t + EPL - 1 in acc[h][0 .. EPL - 1]
    reduce_scatter_step<8, 32>(acc[h]);
    reduce_scatter_step<4, 16>(acc[h]);
    reduce_scatter_step<2, 8>(acc[h]);
    if constexpr (TOK == 16) reduce_scatter_step<1, 4>(acc[h]);
  }

  // ---- merge the 4 waves through LDS (reusing the ring) and write ----
  // Token lane t writes the sums of elements EPL t .. EPL t + EPL - 1 of each
  // head (EPL = 16 / TOK), which are consecutive channels.
  __syncthreads();
  float* sm_acc = reinterpret_cast<float*>(smem);  // [4][GH][D]
  float(*sm_m)[GH] = reinterpret_cast<float(*)[GH]>(sm_acc + 4 * GH * D);  // [4][GH]
  float(*sm_l)[GH] = sm_m + 4;
  {
    constexpr int EPL = 16 / TOK;  // elements per lane: 2 at D 128, 1 at D 64
    static_assert(EPL == 1 || EPL == 2, "lane groups");
#pragma unroll
    for (int h = 0; h < GH; ++h) {
      const int e0 = EPL * t;  // a run of EPL channels inside one chunk of E
      float* dst = sm_acc + (wave * GH + h) * D + E * ((e0 / E) * C + c) + e0 % E;
      if constexpr (EPL == 2) {
        *reinterpret_cast<float2*>(dst) = float2{acc[h][0], acc[h][1]};
      } else {
        *dst = acc[h][0];
      }
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < GH; ++h) {
      sm_m[wave][h] = mw[h];
      sm_l[wave][h] = lsum[h];
    }
  }
  __syncthreads();
  // 4 consecutive outputs per thread: one 16-byte LDS read per wave and one
  // 16-byte store
  for (int idx = threadIdx.x; idx < GH * D / 4; idx += 256) {
    const int h = idx / (D / 4), d = 4 * (idx % (D / 4));
    float M = kNegInf;
#pragma unroll
    for (int wv = 0; wv < 4; ++wv) M = fmaxf(M, sm_m[wv][h]);
    float tot = 0.f;
    float4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int wv = 0; wv < 4; ++wv) {
      const float mwv = sm_m[wv][h];
      if (mwv != kNegInf) {
        const float f = fast_exp2(mwv - M);
        const float4 x = *reinterpret_cast<const float4*>(sm_acc + (wv * GH + h) * D + d);
        tot = fmaf(sm_l[wv][h], f, tot);
        o.x = fmaf(x.x, f, o.x), o.y = fmaf(x.y, f, o.y), o.z = fmaf(x.z, f, o.z), o.w = fmaf(x.w, f, o.w);
      }
    }
    const float inv = tot > 0.f ? 1.f / tot : 0.f;  // 0: every token of the split masked for this row
    o.x *= inv, o.y *= inv, o.z *= inv, o.w *= inv;
    if constexpr (KV == kI8) {
      // P V ran on (1024 + byte ^ 0x80): x_hat = (byte + offset) * scale
      const int vq = a.aq_stride_kv + g * a.aq_stride_g + d * a.aq_stride_d;  // V parameters (index 1)
      const int sd = a.aq_stride_d;
      const float* vsc = a.aq_scale + vq;
      const float* vof = a.aq_offset + vq;
      o.x = vsc[0] * (o.x - 1152.f + vof[0]), o.y = vsc[sd] * (o.y - 1152.f + vof[sd]);
      o.z = vsc[2 * sd] * (o.z - 1152.f + vof[2 * sd]), o.w = vsc[3 * sd] * (o.w - 1152.f + vof[3 * sd]);
    }
    const int64_t row = qrow_of(h);
    *reinterpret_cast<float4*>(a.ws_o + (row * a.n_split + split) * D + d) = o;
    if (d == 0) {
      a.ws_m[row * a.n_split + split] = M * kLn2;
      a.ws_l[row * a.n_split + split] = tot;
    }
  }
}

template <int QT, int KV, int D, int GH>
hipError_t launch_typed(const GqaLaunch& p, hipStream_t stream, const LaunchEvents* ev) {
  const int items = p.batch * p.n_kv * (p.rows_kv / GH) * p.n_split;
  if (items == 0) return hipSuccess;
  // head-group interleave (see the kernel): items without the head group,
  // rounded up to a multiple of 8, times the head groups
  const int padded = (items / (p.rows_kv / GH) + 7) / 8 * 8 * (p.rows_kv / GH);
  if (p.paged)
    launch_kernel(gqa_splitkv_kernel<QT, KV, D, GH, true>, dim3(padded), dim3(256), stream, ev, p, items);
  else
    launch_kernel(gqa_splitkv_kernel<QT, KV, D, GH, false>, dim3(padded), dim3(256), stream, ev, p, items);
  return hipGetLastError();
}

template <int QT, int KV, int D>
hipError_t launch_gh(const GqaLaunch& p, hipStream_t stream, const LaunchEvents* ev) {
  switch (p.heads_per_wg) {
    case 1: return launch_typed<QT, KV, D, 1>(p, stream, ev);
    case 2: return launch_typed<QT, KV, D, 2>(p, stream, ev);
    case 4: return launch_typed<QT, KV, D, 4>(p, stream, ev);
    case 8:
      if constexpr (KV == kF16 || KV == kBF16) return launch_typed<QT, KV, D, 8>(p, stream, ev);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

template <int QT, int KV>
hipError_t launch_d(const GqaLaunch& p, hipStream_t stream, const LaunchEvents* ev) {
  switch (p.head_dim) {
    case 64: return launch_gh<QT, KV, 64>(p, stream, ev);
    case 128: return launch_gh<QT, KV, 128>(p, stream, ev);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int gqa_max_heads_per_wg(int kv_dtype, int head_dim) {
  (void)head_dim;
  // int8 and f32 stop at 4: with 8 the int8 kernel drops to one wave per SIMD
  // and runs slower than two workgroups of 4 heads that share K/V through L2
  return (kv_dtype == kF16 || kv_dtype == kBF16) ? 8 : 4;
}

bool gqa_supported(int q_dtype, int kv_dtype, int head_dim, int heads_per_wg) {
  if (head_dim != 64 && head_dim != 128) return false;
  if (heads_per_wg != 1 && heads_per_wg != 2 && heads_per_wg != 4 && heads_per_wg != 8) return false;
  if (heads_per_wg > gqa_max_heads_per_wg(kv_dtype, head_dim)) return false;
  if (kv_dtype == kI8) return q_dtype == kF32 || q_dtype == kF16 || q_dtype == kBF16;
  return q_dtype == kv_dtype && (kv_dtype == kF32 || kv_dtype == kF16 || kv_dtype == kBF16);
}

hipError_t launch_gqa_splitkv(const GqaLaunch& p, hipStream_t stream, const LaunchEvents* ev) {
  if (!gqa_supported(p.q_dtype, p.kv_dtype, p.head_dim, p.heads_per_wg)) return hipErrorInvalidValue;
  if (p.kv_dtype == kI8) {
    switch (p.q_dtype) {
      case kF32: return launch_d<kF32, kI8>(p, stream, ev);
      case kF16: return launch_d<kF16, kI8>(p, stream, ev);
      default: return launch_d<kBF16, kI8>(p, stream, ev);
    }
  }
  switch (p.kv_dtype) {
    case kF32: return launch_d<kF32, kF32>(p, stream, ev);
    case kF16: return launch_d<kF16, kF16>(p, stream, ev);
    default: return launch_d<kBF16, kBF16>(p, stream, ev);
  }
}

}  // namespace ifa
