// Multi-token GQA split-KV decode on the matrix cores (gfx950).
//
// Speculative verification decodes S_q query tokens per sequence (the last
// S_q of its length) under the masks of the FusedInferAttentionScore pages
// (sparseMode 3 rightDownCausal, 9 treeMask).  A KV head then serves S_q * G
// query rows, and every cached token meets all of them: QK^T and PV become
// dense contractions with M = rows, which this kernel runs on
// v_mfma_f32_32x32x16_{bf16,f16} and writes the split partial triples
// (aclnnRingAttentionUpdate, "功能说明") that the combine kernel merges.
//
// Work decomposition.  One workgroup = one wave = one (KV head, group of up
// to 32 rows) over either one split of one sequence, or, in the balanced
// split, one run of the batch's tiles (equal runs of the tiles of all
// sequences in turn; a run takes one piece of each sequence it touches and
// writes a partial per piece).  Rows are query token major.  A piece's
// tokens stream in tiles of 32 through a private LDS ring of 2 slots,
// each slot the tile's K rows then its V rows (8 KB each for 16-bit K/V, 4 KB
// for int8), loaded straight from HBM with global_load_lds_dwordx4.  Per tile:
//   S^T (32 tokens x 32 rows) = K (32 x 128) . Q^T (128 x 32): 8 MFMAs, K from
//       LDS (ds_read_b128), Q^T in registers for the item;
//   online softmax per row (a lane holds one row column and 16 tokens), the
//       tail of the split and the masks' removed draft tokens at -inf, with
//       the lazy rescale of the other kernels;
//   O^T (128 x 32) += V^T (128 x 32 tokens) . P^T: 8 MFMAs, V^T through the
//       transposing read ds_read_b64_tr_b16, P^T from the S^T accumulator
//       rounded to the K/V dtype (normalised by the sum of the rounded
//       weights; the partial's sum uses the fp32 weights).
// The operand and accumulator layouts are those of the MLA kernel, on
// 256-byte rows: row t keeps its 16-byte chunk c at position c ^ swz16(t)
// (swz(t) on the 128-byte rows of an int8 tile).
//
// int8 K/V (antiquant x_hat = (x + offset) * scale, per channel or per
// tensor): the stored bytes become the exact fp16 values 1152 + x with one
// byte permute (fp16 has unit spacing in [1024, 2048)), so both products run
// on fp16 MFMAs.  The K scale is folded into q (q' = q * scale_K, rounded to
// fp16) and the K offset into a per-row constant sum_d q'_d (offset_d - 1152);
// V^T operands come from the int8 tile through the byte-transposing read
// (ds_read_b64_tr_b8) and are widened in registers, and the V scale and
// offset are applied to the normalised output.
#include "common.hpp"
#include "kernels.hpp"

namespace ifa {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) short s16x4_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

constexpr int kD = 128;
constexpr int kTile = 32;                // tokens per tile
constexpr int kRowB16 = kD * 2;          // bytes of a 16-bit row
constexpr float kRescale = 8.f;
constexpr float kMrefInit = -1e30f;
constexpr int kBalChunks = kLongestFirstMaxBatch / 64;  // sequences per lane in the balanced split

template <int KV, bool TOK>
struct SpecShape {
  static constexpr int ESZ = KV == kI8 ? 1 : 2;
  // tiles in the ring: one tile is computed while the next one loads (a
  // third slot, two tiles in flight, measured slower for both widths)
  static constexpr int STAGES = 2;
  static constexpr int RB = kD * ESZ;       // bytes of one token row of one KV head
  static constexpr int CPR = RB / 16;       // 16-byte chunks per row
  static constexpr int TB = kTile * RB;     // bytes of the K (and of the V) tile
  static constexpr int LT = TB / 1024;      // DMA instructions per K (and per V) tile
  // per-token antiquant: the tile's K scale, K offset, V scale and V offset
  // (32 fp32 each) follow K and V in the slot
  static constexpr int PB = TOK ? 4 * kTile * 4 : 0;
  static constexpr int SLOT = 2 * TB + PB;  // K, V, then the per-token parameters
  static constexpr int SMEM = STAGES * SLOT;
  static constexpr int MK = KV == kBF16 ? kBF16 : kF16;  // MFMA operand type
  static_assert(2 * LT * (STAGES - 1) <= 63 && STAGES >= 2 && STAGES <= 3, "vmcnt, ring");
};

// Row t of an int8 tile (8 chunks of 16 bytes, 128-byte rows: rows of one
// parity share a bank half) keeps chunk c at position c ^ swz(t):
//   - 16 consecutive rows from a multiple of 16 take 8 values per parity (the
//     S^T operand reads: 16 rows, one chunk);
//   - bit 4 of t flips bit 1, so the rows 4 kg + 0..3 and 16 + 4 kg + 0..3 of
//     two neighbouring groups kg (a 32-lane phase of the transposing V^T read
//     in 16 columns; in 32 columns, rows r and 8 + r with two chunks) also
//     take 16 different 16-byte bank groups.
__device__ __forceinline__ int swz(int t) {
  return (2 * (t & 3) + ((t >> 2) & 1)) ^ (2 * ((t >> 3) & 1)) ^ (2 * ((t >> 4) & 1));
}

// Row t of a 16-bit tile (16 chunks, 256 bytes: every row starts in LDS bank
// 0) keeps chunk c at position c ^ swz16(t), with swz16 the bit order of
// t mod 16 reversed and bit 0 also folded into the lowest bit:
//   - 16 consecutive rows take 16 different positions (the S^T operand reads,
//     16 rows per 16-lane phase);
//   - 8 consecutive rows (from a multiple of 8) differ in swz16 / 2, and 4
//     consecutive rows (from a multiple of 4) in swz16 / 4 (the transposing
//     V^T reads: 8 rows x 2 chunks, or 4 rows x 4 chunks, per 32-lane phase);
// So none of these accesses meets another in one bank (a 3-bit swizzle left
// each of them two-way conflicted).
__device__ __forceinline__ int swz16(int t) {
  return 8 * (t & 1) + 4 * ((t >> 1) & 1) + 2 * ((t >> 2) & 1) + (((t >> 3) ^ t) & 1);
}

__device__ __forceinline__ void dma16_lane(const void* src, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, off offset:0 nt" ::"v"(src), "{m0}"(lds) : "memory");
}

// A wave-uniform address in scalar registers, read from the first active
// lane (whatever the compiler made of it).  That read is a VALU write of the
// SGPRs, and a vector memory instruction may read an SGPR only 5 wait states
// after a VALU wrote it; the compiler inserts such waits before its own
// instructions but not before inline asm.  So the address passes through an
// asm that holds the wait and names it as an operand: every load that uses
// the result comes after the wait.
__device__ __forceinline__ const void* sgpr_base(const void* base) {
  const uint64_t x = reinterpret_cast<uint64_t>(base);
  const void* u = reinterpret_cast<const void*>(((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(x >> 32)) << 32) |
                                                (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)x));
  asm volatile("s_nop 4" : "+s"(u));
  return u;
}

// The same as dma16_lane, from a base in scalar registers (sgpr_base) plus a
// 32-bit per-lane byte offset.
__device__ __forceinline__ void dma16_off(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, %1 offset:0 nt" ::"v"(voff), "s"(sbase), "{m0}"(lds) : "memory");
}

// 4 bytes per lane, lane l's at LDS byte address lds + 4 l
__device__ __forceinline__ void dma4_lane(const void* src, uint32_t lds) {
  asm volatile("global_load_lds_dword %0, off offset:0" ::"v"(src), "{m0}"(lds) : "memory");
}

__device__ __forceinline__ f32x4_t lds_read_f32x4(uint32_t addr) {
  return *(const __attribute__((address_space(3))) f32x4_t*)(uintptr_t)addr;
}

template <int N>
__device__ __forceinline__ void wait_vmem() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <typename T>
__device__ __forceinline__ void settle(const T& x) {
  asm volatile("" ::"v"(x));
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

__device__ __forceinline__ u32x4 lds_read_b128(uint32_t addr) {
  return *(const __attribute__((address_space(3))) u32x4*)(uintptr_t)addr;
}

typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

__device__ __forceinline__ u32x2 lds_read_b64(uint32_t addr) {
  return *(const __attribute__((address_space(3))) u32x2*)(uintptr_t)addr;
}

__device__ __forceinline__ void lds_write_b128(uint32_t addr, const u32x4& v) {
  *(__attribute__((address_space(3))) u32x4*)(uintptr_t)addr = v;
}

__device__ __forceinline__ s16x4_t lds_read_tr16(uint32_t addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)(uintptr_t)addr);
}

// Transposing read of bytes: in each 16-lane group, source lane s names 8
// bytes (row s / 2, columns 8 (s % 2) .. + 7 of an 8-row x 16-column block),
// and lane i receives column i of the block, byte j from row j.
__device__ __forceinline__ u32x2 lds_read_tr8(uint32_t addr) {
  typedef __attribute__((ext_vector_type(2))) int i32x2;
  const i32x2 r = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2*)(uintptr_t)addr);
  return u32x2{(uint32_t)r[0], (uint32_t)r[1]};
}

// 32x32x16 MFMA on 16-bit operands held as raw 16-byte vectors
template <int KV>
__device__ __forceinline__ f32x16_t mfma(const u32x4& x, const u32x4& y, const f32x16_t& c) {
  if constexpr (KV == kBF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, x), __builtin_bit_cast(bf16x8_t, y), c,
                                                   0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, x), __builtin_bit_cast(f16x8_t, y), c,
                                                  0, 0, 0);
}

// 16x16x32 MFMA on 16-bit operands held as raw 16-byte vectors
template <int KV>
__device__ __forceinline__ f32x4_t mfma16(const u32x4& x, const u32x4& y, const f32x4_t& c) {
  if constexpr (KV == kBF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, x), __builtin_bit_cast(bf16x8_t, y), c,
                                                   0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, x), __builtin_bit_cast(f16x8_t, y), c,
                                                  0, 0, 0);
}

// Accumulator tile of the NC-column layout: 32x32 (16 registers) or 16x16 (4)
template <int NC>
struct Acc;
template <>
struct Acc<32> {
  typedef f32x16_t type;
};
template <>
struct Acc<16> {
  typedef f32x4_t type;
};

template <int NC, int KV>
__device__ __forceinline__ typename Acc<NC>::type mfma_nc(const u32x4& x, const u32x4& y,
                                                          const typename Acc<NC>::type& c) {
  if constexpr (NC == 32) return mfma<KV>(x, y, c);
  else return mfma16<KV>(x, y, c);
}

// Sum / max over the lanes that hold the same MFMA column: lanes l ^ 32 (32
// columns), or l ^ 16, l ^ 32, l ^ 48 (16 columns).
template <int NC>
__device__ __forceinline__ float col_sum(float x) {
  if constexpr (NC == 16) x = xor16_sum(x);
  return xor32_sum(x);
}
template <int NC>
__device__ __forceinline__ float col_max(float x) {
  if constexpr (NC == 16) x = xor16_max(x);
  return xor32_max(x);
}

// the 16-bit pattern of `v` rounded to the K/V dtype
template <int KV>
__device__ __forceinline__ uint16_t round16(float v) {
  if constexpr (KV == kBF16) return __builtin_bit_cast(uint16_t, (__bf16)v);
  else return __builtin_bit_cast(uint16_t, (_Float16)v);
}

// In-place scale of one accumulator tile: the multiply keeps each value's
// register, so the rare rescale branch gives the tile no new registers
// (which made the compiler copy it at the join).  VREG: the tile lives in
// ordinary registers, as do the 16-column kernels' MFMA accumulators (at most
// 256 registers, so the compiler picks the MFMAs' ordinary-register form; a
// tile pinned to accumulator registers made it copy O there and back around
// every tile's MFMAs).  The 32-column kernels keep their tiles in
// accumulator registers.
template <bool VREG, typename V>
__device__ __forceinline__ void scale_acc(V& v, float s) {
#pragma unroll
  for (int r = 0; r < (int)(sizeof(V) / sizeof(float)); ++r) {
    float x = v[r];
    if constexpr (VREG) {
      asm volatile("v_mul_f32 %0, %0, %1" : "+v"(x) : "v"(s));
    } else {
      float tmp;
      asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                   : "+a"(x), "=&v"(tmp)
                   : "v"(s));
    }
    v[r] = x;
  }
}

// Elements idx .. idx + 7 of a QT array as floats, with 16-byte loads (the
// array 16-byte aligned, idx a multiple of 8) ...
template <int QT>
__device__ __forceinline__ void load8_vec(const void* base, int64_t idx, float (&out)[8]) {
  if constexpr (QT == kF32) {
    const f32x4_t* p = reinterpret_cast<const f32x4_t*>(static_cast<const float*>(base) + idx);
    const f32x4_t x = p[0], y = p[1];
#pragma unroll
    for (int e = 0; e < 4; ++e) out[e] = x[e], out[4 + e] = y[e];
  } else {
    const u32x4 x = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) + idx);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint16_t h = (uint16_t)(word(x, e >> 1) >> (16 * (e & 1)));
      out[e] = QT == kBF16 ? bf16_bits_to_f32(h) : (float)__builtin_bit_cast(_Float16, h);
    }
  }
}
// ... or with element loads
template <int QT>
__device__ __forceinline__ void load8_elem(const void* base, int64_t idx, float (&out)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) out[e] = load_as_f32<QT>(base, idx + e);
}

// int8 bytes of one dword -> the fp16 pairs 1152 + x of bytes (0, 1) and (2, 3)
__device__ __forceinline__ u32x2 widen_i8(uint32_t w) {
  const uint32_t b = w ^ 0x80808080u;
  return u32x2{__builtin_amdgcn_perm(0x64646464u, b, 0x04010400u), __builtin_amdgcn_perm(0x64646464u, b, 0x04030402u)};
}

// BAL: the balanced split (a.balanced), a kernel of its own so that the
// per-sequence kernel stays a single piece.  The 16-column kernels are
// bounded to 256 registers (two waves per SIMD; the 16-bit ones are held to
// one by their LDS anyway), under which the compiler keeps MFMA accumulators
// in ordinary registers.
template <int QT, int KV, bool PAGED, bool TOK, int NC, bool BAL>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(NC == 16 ? 2 : 1)))
gqa_mfma_kernel(const GqaLaunch a, int work_items) {
  using S = SpecShape<KV, TOK>;
  constexpr int RB = S::RB, CPR = S::CPR, TB = S::TB, LT = S::LT, SLOT = S::SLOT, MK = S::MK;
  constexpr int kStages = S::STAGES;
  constexpr bool I8 = KV == kI8;
  // NC query rows per wave in the MFMA columns: 32 (32x32x16 MFMAs) or 16
  // (16x16x32, for KV heads with at most 16 query rows)
  constexpr int KSTEP = NC == 32 ? 16 : 32;  // channels per S^T k-step
  constexpr int NKS = kD / KSTEP;            // S^T k-steps
  constexpr int AW = NC == 32 ? 16 : 4;      // registers per accumulator tile
  constexpr int NSA = kTile / NC;            // S^T tiles per 32-token tile
  constexpr int NSV = NSA * AW;              // scores per lane and tile
  constexpr int TS = NC == 32 ? 8 : 16;      // token step between register quads
  constexpr int NOT = kD / NC;               // O^T tiles
  typedef typename Acc<NC>::type AccT;
  __shared__ __attribute__((aligned(16))) char ring[S::SMEM];

  const int lane = threadIdx.x;

  // ---- work item: (row group, split or run, KV head[, sequence rank]) ----
  const int HG = (a.rows_kv + NC - 1) / NC;
  int rem = blockIdx.x;
  if (rem >= work_items) return;
  const int hg = rem % HG;
  rem /= HG;
  const int split = rem % a.n_split;  // the run, in the balanced split
  rem /= a.n_split;
  const int g = rem % a.n_kv;
  rem /= a.n_kv;

  // The pieces (sequence, token range) this workgroup reduces.  Per-sequence
  // split: one, split `split` of the sequence of rank `rem`.  Balanced split:
  // run `split` of the batch's tiles, which may end one sequence, take short
  // ones whole and start another: one piece per sequence it touches.
  int b = 0, L = 0, start = 0, end = 0;
  int64_t pbase = 0;  // partial of query token qi, head h: pbase + (qi n_q + h) pstride
  int pstride = 1;
  // balanced split: lane l holds, for sequence 64 k + l, the cost of the
  // sequences up to it (inclusive prefix) and its clamped length; the run
  // takes the cost units [tcur, trun_end) of ttotal
  int incl[kBalChunks] = {}, lenv[kBalChunks] = {};
  int nrun = 0, tcur = 0, trun_end = 0, ttotal = 0;
  auto at = [&](const int (&v)[kBalChunks], int idx) -> int {  // entry of sequence idx (wave-uniform)
    const int k = idx >> 6, l = idx & 63;
    int x = __builtin_amdgcn_readlane(v[0], l);
#pragma unroll
    for (int c = 1; c < kBalChunks; ++c) x = k == c ? __builtin_amdgcn_readlane(v[c], l) : x;
    return x;
  };
  if constexpr (!BAL) {
    b = rem;
    if (a.longest_first) {  // the keys use the ring, which no load has reached yet
      const BatchPick pick = batch_of_rank(rem, a.seq_lens, a.batch, a.s_cap, reinterpret_cast<uint32_t*>(ring));
      b = pick.b;
      L = pick.len;
    } else {
      const int64_t L64 = a.seq_lens[b];
      L = (int)(L64 < 0 ? 0 : (L64 > a.s_cap ? a.s_cap : L64));
    }
    const int per = (int)split_chunk(L, a.n_split);
    start = split * per;
    end = min(L, start + per);
    if (start >= end) return;  // empty split: nothing is written for it
    pbase = (int64_t)b * a.q_seq * a.n_q * a.n_split + split;
    pstride = a.n_split;
  } else {
    // Cost of a sequence: its tiles plus kGqaPieceCost for the start of a
    // piece on it; none for an empty one.
    int carry = 0;
#pragma unroll
    for (int k = 0; k < kBalChunks; ++k) {
      if (64 * k >= a.batch) {  // wave-uniform: no sequences in this chunk
        incl[k] = carry;
        continue;
      }
      const int bb = 64 * k + lane;
      int Lb = 0;
      if (bb < a.batch) {
        const int64_t L64 = a.seq_lens[bb];
        Lb = (int)(L64 < 0 ? 0 : (L64 > a.s_cap ? a.s_cap : L64));
      }
      int t = Lb > 0 ? (Lb + kTile - 1) / kTile + kGqaPieceCost : 0;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(t, d);
        if (lane >= d) t += y;
      }
      incl[k] = carry + t;
      lenv[k] = Lb;
      carry += __builtin_amdgcn_readfirstlane(__shfl(t, 63));  // the chunk's total, in a scalar register
    }
    ttotal = carry;
    // runs: min(n_split, total cost) of them, so that none is empty; run r
    // covers cost units [r V / R, (r + 1) V / R) (floors)
    nrun = min(a.n_split, ttotal);
    if (split >= nrun) return;
    tcur = (int)((int64_t)split * ttotal / nrun);
    trun_end = (int)((int64_t)(split + 1) * ttotal / nrun);
    // the sequence holding unit tcur: as many as have a prefix <= tcur precede it
    int before = 0;
#pragma unroll
    for (int k = 0; k < kBalChunks; ++k)
      before += __builtin_popcountll(__builtin_amdgcn_ballot_w64(64 * k + lane < a.batch && incl[k] <= tcur));
    b = before;
  }

  for (;;) {
    if constexpr (BAL) {
      // sequence b spans units [pb, pe): kGqaPieceCost for its start, then
      // one per tile from z on.  The run's units hold its tiles
      // [max(tcur, z), min(trun_end, pe)) - z; none when the run ends inside
      // the start units (the next run takes the sequence).
      const int pb = b == 0 ? 0 : at(incl, b - 1);
      const int pe = at(incl, b);
      const int z = pb + kGqaPieceCost;
      if (trun_end <= z) break;
      const int first = max(tcur, z);
      L = at(lenv, b);
      start = (first - z) * kTile;
      end = min(L, (min(trun_end, pe) - z) * kTile);
      pbase = (int64_t)(split + b) * a.q_seq * a.n_q;
      pstride = 1;
      if (first == z && g == 0 && hg == 0 && lane == 0) {
        // the runs that take sequence b are this one .. the one holding its last unit
        const int rlast = (int)(((int64_t)pe * nrun - 1) / ttotal);
        a.seg_desc[b] = make_int2(split + b, rlast - split + 1);
      }
    }
    const int ntiles = (end - start + kTile - 1) / kTile;
    // This lane, made opaque for each piece in the balanced split: what
    // derives from it (LDS offsets, channels, rows) is then computed per piece
    // instead of being hoisted out of the piece loop and held across it.
    int lane_p = lane;
    if constexpr (BAL) asm volatile("" : "+v"(lane_p));
    const int kg = lane_p / NC;  // which group of 8 k-slots of an MFMA this lane feeds
    const int col = lane_p % NC;
    // The antiquant parameters, read afresh for each piece: hoisted out of
    // the piece loop, the per-channel ones would hold 128 registers across
    // it.  Only the KV head's offset into them is made opaque per piece, so
    // that their loads stay global loads.
    const float* aq_scale = a.aq_scale;
    const float* aq_offset = a.aq_offset;
    int aq_g = __builtin_amdgcn_readfirstlane(g * a.aq_stride_g);  // the KV head's parameters
    if constexpr (BAL) asm volatile("" : "+s"(aq_g));

    // ---- this lane's row (the MFMA column it holds), its mask over the drafts ----
    const int rr = hg * NC + col;  // row of the KV head's q_seq * group rows
    const bool row_ok = rr < a.rows_kv;
    const int qi = row_ok ? rr / a.group : 0;
    const int hrow = g * a.group + (row_ok ? rr - qi * a.group : 0);  // query head
    const int64_t qrow = ((int64_t)b * a.q_seq + qi) * a.n_q + hrow;
    const int64_t pidx = pbase + ((int64_t)qi * a.n_q + hrow) * pstride;  // this row's partial
    const int draft0 = L - a.q_seq;  // position of draft token 0
    uint32_t vis = ~0u;  // bit k: the row attends to draft token k
    if (a.mask_mode == 3) {
      vis = (2u << qi) - 1u;
    } else if (a.mask_mode == 9) {
      // the row's q_seq <= 16 mask bytes, all loaded (at clamped, in-bounds
      // positions) before any is used
      const uint8_t* m = a.tree_mask + ((int64_t)b * a.q_seq + qi) * a.q_seq;
      uint8_t mk[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) mk[k] = m[min(k, a.q_seq - 1)];
      vis = 0;
#pragma unroll
      for (int k = 0; k < 16; ++k) vis |= (k < a.q_seq && mk[k] == 0 ? 1u : 0u) << k;
    }

    // ---- Q^T operand: channels KSTEP ks + 8 kg .. + 7 per k-step (zero for padding rows) ----
    u32x4 qreg[NKS];
    float kconst = 0.f;  // int8: sum_d q'_d (offset_d - 1152) over the row
    float qsum = 0.f;    // per-token int8: sum_d q_d of the fp16 query
    if constexpr (I8 && !TOK && NC == 32) {
      // q' = q * scale_K rounded to fp16, and this lane's half of the constant,
      // element by element: the batched form below, with 64 channels per
      // lane here, took this kernel past the 256 registers of two waves per
      // SIMD
      float part = 0.f;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          uint32_t pair = 0;
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int d = KSTEP * ks + 8 * kg + 2 * w + e;
            const int kq = aq_g + d * a.aq_stride_d;  // K parameters (index 0)
            const _Float16 qh = row_ok ? (_Float16)(load_as_f32<QT>(a.q, qrow * kD + d) * aq_scale[kq]) : (_Float16)0.f;
            part = fmaf((float)qh, aq_offset[kq] - 1152.f, part);
            pair |= (uint32_t)__builtin_bit_cast(uint16_t, qh) << (16 * e);
          }
          qreg[ks][w] = pair;
        }
      kconst = col_sum<NC>(part);  // the lanes of one column hold its channels between them
    } else if constexpr (I8) {
      // Channels KSTEP ks + 8 kg .. + 7 of the row, and (per channel) their K
      // parameters, CH k-steps at a time: each chunk's loads are all issued
      // before any is used, unconditionally (a padding row reads a valid row
      // and is zeroed after), so a chunk costs one memory round trip rather
      // than one per element.  (16 columns: one chunk of 4 k-steps, 96
      // registers; 32 columns: four of 2 k-steps, which keeps the kernel at
      // two waves per SIMD.)
      constexpr int CH = NC == 16 ? 4 : 2;
      const bool qvec = (reinterpret_cast<uintptr_t>(a.q) & 15) == 0;
      const bool pchan = a.aq_stride_d == 1;  // per channel (2, N_kv, D); else per tensor (2)
      const bool pvec = ((reinterpret_cast<uintptr_t>(aq_scale) | reinterpret_cast<uintptr_t>(aq_offset)) & 15) == 0;
      float part = 0.f;
#pragma unroll
      for (int c0 = 0; c0 < NKS; c0 += CH) {
        float qf[CH][8], sc[TOK ? 1 : CH][8], of[TOK ? 1 : CH][8];
        if (qvec) {
#pragma unroll
          for (int k = 0; k < CH; ++k) load8_vec<QT>(a.q, qrow * kD + KSTEP * (c0 + k) + 8 * kg, qf[k]);
        } else {
#pragma unroll
          for (int k = 0; k < CH; ++k) load8_elem<QT>(a.q, qrow * kD + KSTEP * (c0 + k) + 8 * kg, qf[k]);
        }
        if constexpr (!TOK) {
          if (pchan && pvec) {
#pragma unroll
            for (int k = 0; k < CH; ++k) {
              load8_vec<kF32>(aq_scale, aq_g + KSTEP * (c0 + k) + 8 * kg, sc[k]);
              load8_vec<kF32>(aq_offset, aq_g + KSTEP * (c0 + k) + 8 * kg, of[k]);
            }
          } else if (pchan) {
#pragma unroll
            for (int k = 0; k < CH; ++k) {
              load8_elem<kF32>(aq_scale, aq_g + KSTEP * (c0 + k) + 8 * kg, sc[k]);
              load8_elem<kF32>(aq_offset, aq_g + KSTEP * (c0 + k) + 8 * kg, of[k]);
            }
          } else {
            const float s0 = aq_scale[aq_g], o0 = aq_offset[aq_g];
#pragma unroll
            for (int k = 0; k < CH; ++k)
#pragma unroll
              for (int e = 0; e < 8; ++e) sc[k][e] = s0, of[k][e] = o0;
          }
        }
#pragma unroll
        for (int k = 0; k < CH; ++k)
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            uint32_t pair = 0;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              const int j = 2 * w + e;
              _Float16 qh;
              if constexpr (TOK) {
                // q in fp16 as given (the K scale varies per token and multiplies the score)
                qh = row_ok ? (_Float16)qf[k][j] : (_Float16)0.f;
                part += (float)qh;
              } else {
                // q' = q * scale_K rounded to fp16, and this lane's part of the constant
                qh = row_ok ? (_Float16)(qf[k][j] * sc[k][j]) : (_Float16)0.f;
                part = fmaf((float)qh, of[k][j] - 1152.f, part);
              }
              pair |= (uint32_t)__builtin_bit_cast(uint16_t, qh) << (16 * e);
            }
            qreg[c0 + k][w] = pair;
          }
        // the scheduler would otherwise pull the next chunk's loads up here
        __builtin_amdgcn_sched_barrier(0);
      }
      // the lanes of one column hold its channels between them
      if constexpr (TOK) qsum = col_sum<NC>(part);
      else kconst = col_sum<NC>(part);
    } else if ((reinterpret_cast<uintptr_t>(a.q) & 15) == 0) {  // 16-byte loads
      // loaded unconditionally (a padding row reads a valid row) and zeroed after
      const u32x4* qp = reinterpret_cast<const u32x4*>(static_cast<const char*>(a.q) + qrow * RB) + kg;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) qreg[ks] = qp[KSTEP / 8 * ks];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int w = 0; w < 4; ++w) qreg[ks][w] = row_ok ? word(qreg[ks], w) : 0u;
    } else {  // a query buffer aligned to its element only
      const uint16_t* qp = reinterpret_cast<const uint16_t*>(static_cast<const char*>(a.q) + qrow * RB) + 8 * kg;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t v = (uint32_t)qp[KSTEP * ks + 2 * w] | ((uint32_t)qp[KSTEP * ks + 2 * w + 1] << 16);
          qreg[ks][w] = row_ok ? v : 0u;
        }
    }
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) settle(qreg[ks]);
    settle(kconst);
    settle(qsum);

    // per-token antiquant: rows of this sequence (and KV head) in the K scale,
    // K offset, V scale and V offset arrays
    const float* tokp[4] = {nullptr, nullptr, nullptr, nullptr};
    if constexpr (TOK) {
      const int64_t base = (int64_t)b * a.aq_tok_stride_b + (int64_t)g * a.aq_tok_stride_g;
      tokp[0] = aq_scale + base;
      tokp[1] = aq_offset + base;
      tokp[2] = aq_scale + a.aq_tok_stride_kv + base;
      tokp[3] = aq_offset + a.aq_tok_stride_kv + base;
    }

    // ---- block-table slice of the split: lane k holds its k-th block id ----
    const uint32_t bi_first = PAGED ? fast_div((uint32_t)start, a.bs_magic, a.bs_shift) : 0;
    int tbl = 0;
    if constexpr (PAGED) {
      const int nblk = (int)fast_div((uint32_t)(end - 1), a.bs_magic, a.bs_shift) - (int)bi_first + 1;
      tbl = lanes_from_scalar_loads(a.block_table + (int64_t)b * a.max_blocks + bi_first, nblk < 64 ? nblk : 64, 0);
    }
    auto block_id = [&](uint32_t bi) -> uint32_t {  // wave-uniform
      const uint32_t k = bi - bi_first;
      int v = k < 64 ? __builtin_amdgcn_readlane(tbl, k) : ld_uniform(a.block_table, (int64_t)b * a.max_blocks + bi);
      return (uint32_t)(v < 0 ? 0 : (v >= a.num_blocks ? a.num_blocks - 1 : v));
    };

    const char* kbase = static_cast<const char*>(a.k);
    const char* vbase = static_cast<const char*>(a.v);
    const uint32_t ring_lds = lds_addr(ring);

    // per-lane rows of the tile starting at token tstart into LDS byte address dst
    auto queue_rows = [&](int tstart, uint32_t dst) {
      uint32_t tok0 = 0, adj0 = 0, adj1 = 0, adj2 = 0;
      if constexpr (PAGED) {
        const uint32_t bi0 = fast_div((uint32_t)tstart, a.bs_magic, a.bs_shift);
        const uint32_t bil = fast_div((uint32_t)(end - 1), a.bs_magic, a.bs_shift);
        tok0 = bi0 * (uint32_t)a.block_size;
        adj0 = block_id(bi0);
        adj1 = block_id(bi0 + 1 <= bil ? bi0 + 1 : bil);
        adj2 = block_id(bi0 + 2 <= bil ? bi0 + 2 : bil);
      }
#pragma unroll
      for (int i = 0; i < LT; ++i) {
        const int P = 64 * i + lane_p;
        const int t = P / CPR;
        const int c = (P % CPR) ^ (I8 ? swz(t) : swz16(t));
        const uint32_t tok = (uint32_t)min(tstart + t, end - 1);
        uint64_t row;
        if constexpr (PAGED) {
          const uint32_t bs = (uint32_t)a.block_size;
          const uint32_t u = tok - tok0;
          const uint32_t blk = u >= 2 * bs ? adj2 : (u >= bs ? adj1 : adj0);
          const uint32_t slot_in = u - (u >= 2 * bs ? 2 * bs : (u >= bs ? bs : 0));
          row = a.token_major ? ((uint64_t)blk * bs + slot_in) * (uint32_t)a.n_kv + (uint32_t)g
                              : ((uint64_t)blk * (uint32_t)a.n_kv + (uint32_t)g) * bs + slot_in;
        } else {
          row = a.token_major ? ((uint64_t)b * (uint64_t)a.s_cap + tok) * (uint32_t)a.n_kv + (uint32_t)g
                              : ((uint64_t)b * (uint32_t)a.n_kv + (uint32_t)g) * (uint64_t)a.s_cap + tok;
        }
        const uint64_t off = row * RB + 16u * (uint32_t)c;
        dma16_lane(kbase + off, dst + 1024 * i);
        dma16_lane(vbase + off, dst + TB + 1024 * i);
      }
    };

    // Queue tile j into ring slot `slot`: LDS chunk position P of the K (or V)
    // tile holds row t = P / CPR, chunk (P % CPR) ^ swz16(t) (int8: swz(t)) of token tstart + t
    // (rows past the split's end repeat its last row).  A tile's 32 tokens lie
    // in at most 3 cache blocks.
    //
    // A whole tile (32 tokens of the piece, in one cache block or in a
    // contiguous cache) is 32 rows at a fixed stride from its first row: lane
    // l's chunk of load i then sits at byte loff[i] from that row, the same
    // for every such tile, and the tile costs a scalar base per K and V and
    // the loads.  Other tiles (straddling a block boundary, or the piece's
    // last) take the per-lane row computation.
    const uint32_t row_stride = a.token_major ? (uint32_t)a.n_kv * RB : (uint32_t)RB;
    uint32_t loff[LT];
#pragma unroll
    for (int i = 0; i < LT; ++i) {
      const int P = 64 * i + lane_p;
      const int t = P / CPR;
      loff[i] = (uint32_t)t * row_stride + 16u * (uint32_t)((P % CPR) ^ (I8 ? swz(t) : swz16(t)));
    }
    auto queue_tile = [&](int j, int slot) {
      const int tstart = start + kTile * j;
      const uint32_t dst = ring_lds + slot * SLOT;
      bool whole = tstart + kTile <= end;
      uint64_t row0 = 0;  // row of token tstart
      if constexpr (PAGED) {
        const uint32_t bs = (uint32_t)a.block_size;
        const uint32_t bi = fast_div((uint32_t)tstart, a.bs_magic, a.bs_shift);
        const uint32_t u = (uint32_t)tstart - bi * bs;
        whole = whole && u + kTile <= bs;
        if (whole) {
          const uint32_t blk = block_id(bi);
          row0 = a.token_major ? ((uint64_t)blk * bs + u) * (uint32_t)a.n_kv + (uint32_t)g
                               : ((uint64_t)blk * (uint32_t)a.n_kv + (uint32_t)g) * bs + u;
        }
      } else {
        row0 = a.token_major ? ((uint64_t)b * (uint64_t)a.s_cap + (uint32_t)tstart) * (uint32_t)a.n_kv + (uint32_t)g
                             : ((uint64_t)b * (uint32_t)a.n_kv + (uint32_t)g) * (uint64_t)a.s_cap + (uint32_t)tstart;
      }
      if (whole) {
        const uint64_t boff = row0 * RB;
        const void* kt = sgpr_base(kbase + boff);
        const void* vt = sgpr_base(vbase + boff);
#pragma unroll
        for (int i = 0; i < LT; ++i) {
          dma16_off(kt, loff[i], dst + 1024 * i);
          dma16_off(vt, loff[i], dst + TB + 1024 * i);
        }
      } else {
        queue_rows(tstart, dst);
      }
      if constexpr (TOK) {
        // parameter array 2 k + (lane / 32), token tstart + lane % 32 (clamped
        // to the split's last token), to slot byte 2 TB + 128 (2 k + lane / 32)
        const int tok = min(tstart + (lane_p & 31), end - 1);
#pragma unroll
        for (int k = 0; k < 2; ++k) dma4_lane((lane_p >> 5 ? tokp[2 * k + 1] : tokp[2 * k]) + tok, dst + 2 * TB + 256 * k);
      }
    };

#pragma unroll
    for (int s = 0; s < kStages - 1; ++s)
      if (s < ntiles) queue_tile(s, s);

    // ---- per-lane LDS offsets within a slot ----
    // S^T A operand of S^T tile m: token t = NC m + col, channels KSTEP ks + 8 kg
    // .. + 7: 16-byte chunk KSTEP ks / 8 + kg of a 16-bit row, or 8 bytes of an
    // int8 row (chunk (KSTEP ks + 8 kg) / 16, half ((KSTEP ks + 8 kg) / 8) % 2)
    uint32_t offS[NSA][NKS];
#pragma unroll
    for (int m = 0; m < NSA; ++m)
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const int t = NC * m + col;
        const int c8 = (KSTEP * ks + 8 * kg) / 8;  // 8-channel group of the row
        offS[m][ks] = I8 ? t * RB + 16 * ((c8 >> 1) ^ swz(t)) + 8 * (c8 & 1) : t * RB + 16 * (c8 ^ swz16(t));
      }
    // V^T A operand (transposing read) on 16-bit rows.  In 16-lane group gq,
    // source lane s = 4 r + q reads 4 channels of
    // one row, the group a 4-row x 16-channel block, and the read hands lane i
    // of the group the 4 tokens of channel i of the block.
    //   32 columns: row 8 rd + 4 (gq / 2) + r, chunk 8 hi + 4 (tile & 1) + 2
    //     (gq & 1) + q / 2 with hi = tile / 2, for the k-slots 4 h + 0..3 (rd 0)
    //     and 8 + 4 h + 0..3 (rd 1) of each 16-token k-step (k-step 1: rows
    //     16 further, an immediate, as the swizzle repeats every 16 rows);
    //   16 columns: row 16 rd + 4 gq + r, chunk 8 hi + 2 (tile & 3) + q / 2
    //     with hi = tile / 4, for the k-slots 0..3 (tokens 4 kg + 0..3) and
    //     4..7 (tokens 16 + 4 kg + 0..3) of the single 32-token k-step.
    // Offsets [hi][tile part][rd]; half q % 2.
    //
    // int8 V: the byte-transposing read takes the same k-slots straight from
    // the int8 tile, 8 tokens per lane.  Source lane s = 2 j + e of group gq
    // names row j of the block (the token of k-slot j) and channels 8 e .. + 7
    // of the MFMA's 16: chunk `tile` (16 columns) or 2 (tile % 4) + (gq & 1)
    // (32 columns), tokens as above; in 32 columns k-step 1 lies 16 rows
    // further, where bit 4 of the row changes the swizzle, so it has offsets
    // of its own.  Offset n belongs to PV MFMA n.
    uint32_t offV[I8 ? 1 : 2][4][2];
    uint32_t offV8[I8 ? 8 : 1];
    if constexpr (I8) {
      const int s = lane_p & 15, gq = lane_p >> 4;
      const int j = s >> 1, e = s & 1;
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        const int kk = NC == 32 ? n / NOT : 0, mt = NC == 32 ? n % NOT : n;
        const int t = NC == 32 ? 16 * kk + 8 * (j >> 2) + 4 * (gq >> 1) + (j & 3) : 16 * (j >> 2) + 4 * gq + (j & 3);
        const int c = NC == 32 ? 2 * mt + (gq & 1) : mt;
        offV8[n] = t * RB + 16 * (c ^ swz(t)) + 8 * e;
      }
    } else {
      const int s = lane_p & 15, gq = lane_p >> 4;
      const int r = s >> 2, q = s & 3;
#pragma unroll
      for (int hi = 0; hi < 2; ++hi)
#pragma unroll
        for (int rd = 0; rd < 2; ++rd)
#pragma unroll
          for (int tp = 0; tp < 4; ++tp) {
            const int t = NC == 32 ? 8 * rd + 4 * (gq >> 1) + r : 16 * rd + 4 * gq + r;
            const int x = 8 * hi + (NC == 32 ? 4 * (tp & 1) + 2 * (gq & 1) + (q >> 1) : 2 * tp + (q >> 1));
            offV[hi][tp][rd] = t * kRowB16 + 16 * (x ^ swz16(t)) + 8 * (q & 1);
          }
    }

    float mref = kMrefInit, mtrue = kNegInf, lsum = 0.f, lsum_r = 0.f;
    float vbias = 0.f;  // per-token int8: sum over tokens of rounded weight * (offset_V - 1152)
    AccT acc[NOT];
#pragma unroll
    for (int mt = 0; mt < NOT; ++mt)
#pragma unroll
      for (int r = 0; r < AW; ++r) acc[mt][r] = 0.f;

    for (int i = 0; i < ntiles; ++i) {
      // tile i has landed once only the loads of the tiles queued after it
      // (at most kStages - 2) remain (vmcnt retires in order)
      const int after = min(kStages - 2, ntiles - 1 - i);
      if constexpr (kStages == 3) {
        if (after >= 1) wait_vmem<2 * LT>();
        else wait_vmem<0>();
      } else {
        wait_vmem<0>();
      }
      // tile i + kStages - 1 goes into the slot of tile i - 1, whose operands
      // this wave read during the last iteration, before their MFMAs.  Queued
      // after the wait: with two slots one tile is in flight while this one is
      // computed, which measured faster than queueing it before the wait (two
      // in flight) or a third slot.
      if (i + kStages - 1 < ntiles) queue_tile(i + kStages - 1, (i + kStages - 1) % kStages);
      const uint32_t slot = ring_lds + (i % kStages) * SLOT;
      const int tstart = start + kTile * i;

      // ---- S^T = K . Q^T ----
      AccT sacc[NSA];
#pragma unroll
      for (int m = 0; m < NSA; ++m)
#pragma unroll
        for (int r = 0; r < AW; ++r) sacc[m][r] = 0.f;
      u32x4 kb[NSA][NKS];
#pragma unroll
      for (int m = 0; m < NSA; ++m)
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          if constexpr (I8) {
            const u32x2 x = lds_read_b64(slot + offS[m][ks]);
            const u32x2 w0 = widen_i8(x[0]), w1 = widen_i8(x[1]);
            kb[m][ks] = u32x4{w0[0], w0[1], w1[0], w1[1]};
          } else {
            kb[m][ks] = lds_read_b128(slot + offS[m][ks]);
          }
        }
      // every K operand read is issued before the first MFMA (left alone, the
      // scheduler put each read next to its MFMA and waited for it there)
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int m = 0; m < NSA; ++m)
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) sacc[m] = mfma_nc<NC, MK>(kb[m][ks], qreg[ks], sacc[m]);

      // ---- online softmax over this lane's row (column) ----
      // score register r (accumulator register r % AW of S^T tile r / AW) holds
      // token TS (r / 4) + 4 kg + r % 4 of the tile
      float sv[NSV];
      if constexpr (TOK) {
        // score of token t: scale_K[t] (q . (1152 + x_t) + (offset_K[t] - 1152) sum q); this lane's
        // tokens TS q4 + 4 kg + e lie in 16-byte groups of each parameter array
        const uint32_t pa = slot + 2 * TB + 16 * kg;
#pragma unroll
        for (int q4 = 0; q4 < NSV / 4; ++q4) {
          const f32x4_t sk = lds_read_f32x4(pa + 4 * TS * q4), ok = lds_read_f32x4(pa + 128 + 4 * TS * q4);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * q4 + e;
            sv[r] = sk[e] * fmaf(ok[e] - 1152.f, qsum, sacc[r / AW][r % AW]) * a.scale_log2;
          }
        }
      } else {
#pragma unroll
        for (int r = 0; r < NSV; ++r) {
          // (16-bit K: no per-row constant; adding 0 is not free in floating point)
          if constexpr (I8) sv[r] = (sacc[r / AW][r % AW] + kconst) * a.scale_log2;
          else sv[r] = sacc[r / AW][r % AW] * a.scale_log2;
        }
      }
      if (tstart + kTile > end || tstart + kTile > draft0) {  // the split's tail, or draft tokens
#pragma unroll
        for (int r = 0; r < NSV; ++r) {
          const int tok = tstart + TS * (r >> 2) + 4 * kg + (r & 3);
          const uint32_t k = (uint32_t)(tok - draft0);  // draft index; huge for tokens before the drafts
          const uint32_t kept = k < 32u ? (vis >> k) & 1u : 1u;
          const uint32_t keep = (uint32_t)(tok < end) & kept;
          sv[r] = keep ? sv[r] : kNegInf;  // a select, not a branch
        }
      }
      float smax = kNegInf;
#pragma unroll
      for (int r = 0; r < NSV; ++r) smax = fmaxf(smax, sv[r]);
      smax = col_max<NC>(smax);  // the column's other tokens sit in the lanes l ^ 16 / 32 / 48
      mtrue = fmaxf(mtrue, smax);
      if (__builtin_amdgcn_ballot_w64(smax > mref + kRescale)) {
        const float mnew = smax > mref + kRescale ? smax : mref;
        const float alpha = fast_exp2(mref - mnew);  // 0 on the first scores
        lsum *= alpha;
        lsum_r *= alpha;
        vbias *= alpha;
#pragma unroll
        for (int mt = 0; mt < NOT; ++mt) scale_acc<NC == 16>(acc[mt], alpha);
        mref = mnew;
      }
      // P^T operand: k-slot j of lane group kg in 16-token k-step kk is score
      // register 8 kk + j (32 columns), or, in the one 32-token k-step, score
      // register j (16 columns), rounded to the MFMA operand type
      u32x4 pb[NSV / 8];
      float pr[NSV];
      float pscale[NSV], pbias[NSV];  // per-token int8: V scale and offset - 1152 of each token
      if constexpr (TOK) {
        const uint32_t pa = slot + 2 * TB + 256 + 16 * kg;
#pragma unroll
        for (int q4 = 0; q4 < NSV / 4; ++q4) {
          const f32x4_t sv4 = lds_read_f32x4(pa + 4 * TS * q4), ov4 = lds_read_f32x4(pa + 128 + 4 * TS * q4);
#pragma unroll
          for (int e = 0; e < 4; ++e) pscale[4 * q4 + e] = sv4[e], pbias[4 * q4 + e] = ov4[e] - 1152.f;
        }
      }
#pragma unroll
      for (int r = 0; r < NSV; ++r) {
        const float pf = fast_exp2(sv[r] - mref);  // <= 2^8; 0 for removed tokens
        lsum += pf;
        // per-token int8: the weight that multiplies the widened V row is
        // p * scale_V[t]; its rounded value also removes the 1152 bias and adds
        // the V offset through vbias
        const uint16_t bits = round16<MK>(TOK ? pf * pscale[r] : pf);
        pr[r] = MK == kBF16 ? (float)__builtin_bit_cast(__bf16, bits) : (float)__builtin_bit_cast(_Float16, bits);
        if (r & 1) pb[r >> 3][(r & 7) >> 1] |= (uint32_t)bits << 16;
        else pb[r >> 3][(r & 7) >> 1] = bits;
      }
      if constexpr (TOK) {
#pragma unroll
        for (int r = 0; r < NSV; ++r) vbias = fmaf(pr[r], pbias[r], vbias);
      } else {
#pragma unroll
        for (int r = 0; r < NSV; ++r) lsum_r += pr[r];
      }

      // ---- O^T += V^T . P^T ----
      // 32 columns: MFMA n takes k-step n / 4 and row tile n % 4 (32 channels);
      // 16 columns: MFMA n takes row tile n (16 channels) over all 32 tokens
      u32x4 vb[8];
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        if constexpr (I8) {
          // 8 tokens of one channel as int8, widened to the fp16 values 1152 + x
          const u32x2 x = lds_read_tr8(slot + TB + offV8[n]);
          const u32x2 w0 = widen_i8(x[0]), w1 = widen_i8(x[1]);
          vb[n] = u32x4{w0[0], w0[1], w1[0], w1[1]};
        } else {
          const int kk = NC == 32 ? n / NOT : 0, mt = NC == 32 ? n % NOT : n;
          const int tp = NC == 32 ? (mt & 1) : (mt & 3);
          const int hi8 = NC == 32 ? (mt >> 1) : (mt >> 2);
          const uint32_t imm = kRowB16 * 16 * kk;
          const s16x4_t lo = lds_read_tr16(slot + TB + offV[hi8][tp][0] + imm);
          const s16x4_t hi = lds_read_tr16(slot + TB + offV[hi8][tp][1] + imm);
          vb[n] = __builtin_bit_cast(u32x4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
      }
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        const int kk = NC == 32 ? n / NOT : 0, mt = NC == 32 ? n % NOT : n;
        acc[mt] = mfma_nc<NC, MK>(vb[n], pb[kk], acc[mt]);
      }
    }

    // ---- partial triple: normalised out, true max, sum relative to it ----
    const float ltot = col_sum<NC>(lsum);
    // normaliser: the rounded weights PV applied (per-channel int8 and 16-bit:
    // this also cancels the 1152 bias exactly), or, per-token, the fp32 weights
    // whose scaled and rounded values PV applied (the bias leaves through vbias)
    const float lr = TOK ? ltot : col_sum<NC>(lsum_r);
    const float inv = lr > 0.f ? 1.f / lr : 0.f;  // 0: every token of the split removed for this row
    const float vb = TOK ? col_sum<NC>(vbias) * inv : 0.f;
#pragma unroll
    for (int mt = 0; mt < NOT; ++mt) scale_acc<NC == 16>(acc[mt], inv);
    // O^T tile mt, register 4 r4 + e: channel NC mt + 8 r4 + 4 kg + e.  int8
    // (per channel or per tensor): the V parameters of a group of G tiles'
    // channels are all loaded before that group's stores (the stores may
    // alias them for the compiler, which would otherwise wait for each load
    // in turn); 16 columns: all 8 tiles at once, 64 registers.
    constexpr int G = NC == 16 ? NOT : 1;
    const float* ps = aq_scale + a.aq_stride_kv + aq_g;
    const float* po = aq_offset + a.aq_stride_kv + aq_g;
    const bool vvec = a.aq_stride_d == 1 && ((reinterpret_cast<uintptr_t>(ps) | reinterpret_cast<uintptr_t>(po)) & 15) == 0;
    float* o = a.ws_o + pidx * kD;
#pragma unroll
    for (int m0 = 0; m0 < NOT; m0 += G) {
      f32x4_t vsc[I8 && !TOK ? G : 1][AW / 4], voff[I8 && !TOK ? G : 1][AW / 4];
      if constexpr (I8 && !TOK) {
        if (vvec) {
#pragma unroll
          for (int m = 0; m < G; ++m)
#pragma unroll
            for (int r4 = 0; r4 < AW / 4; ++r4) {
              const int d = NC * (m0 + m) + 8 * r4 + 4 * kg;
              vsc[m][r4] = *reinterpret_cast<const f32x4_t*>(ps + d);
              voff[m][r4] = *reinterpret_cast<const f32x4_t*>(po + d);
            }
        } else {
#pragma unroll
          for (int m = 0; m < G; ++m)
#pragma unroll
            for (int r4 = 0; r4 < AW / 4; ++r4)
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int d = (NC * (m0 + m) + 8 * r4 + 4 * kg + e) * a.aq_stride_d;
                vsc[m][r4][e] = ps[d];
                voff[m][r4][e] = po[d];
              }
        }
      }
      if (row_ok) {
#pragma unroll
        for (int m = 0; m < G; ++m)
#pragma unroll
          for (int r4 = 0; r4 < AW / 4; ++r4) {
            const int mt = m0 + m;
            const int d = NC * mt + 8 * r4 + 4 * kg;
            f32x4_t v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = acc[mt][4 * r4 + e];
            if constexpr (TOK) {
#pragma unroll
              for (int e = 0; e < 4; ++e) v[e] += vb;
            } else if constexpr (I8) {
              // P V ran on 1152 + x: x_hat = (x + offset) * scale per channel (index 1)
#pragma unroll
              for (int e = 0; e < 4; ++e) v[e] = vsc[m][r4][e] * (v[e] - 1152.f + voff[m][r4][e]);
            }
            *reinterpret_cast<f32x4_t*>(o + d) = v;
          }
      }
    }
    if (row_ok && kg == 0) {
      a.ws_m[pidx] = mtrue * kLn2;
      a.ws_l[pidx] = ltot > 0.f ? ltot * fast_exp2(mref - mtrue) : 0.f;
    }

    // next piece: the next sequence with tiles, while the run lasts
    if constexpr (!BAL) break;
    tcur = min(trun_end, at(incl, b));
    if (tcur >= trun_end) break;
    do {
      ++b;  // stays below batch: units remain after tcur
    } while (at(incl, b) == tcur);
  }
}

template <int QT, int KV, bool TOK, int NC>
hipError_t launch_nc(const GqaLaunch& p, hipStream_t stream, const LaunchEvents* ev) {
  // per-sequence split: (row group, split, KV head, sequence); balanced: (row group, run, KV head)
  const int items = (p.balanced ? 1 : p.batch) * p.n_kv * ((p.rows_kv + NC - 1) / NC) * p.n_split;
  if (items == 0) return hipSuccess;
  if constexpr (KV == kI8 && NC == 32) {
    // the balanced int8 kernel with 32 columns would need more than the 256
    // registers of two waves per SIMD: the host splits such shapes per sequence
    if (p.balanced) return hipErrorInvalidValue;
    launch_kernel(p.paged ? gqa_mfma_kernel<QT, KV, true, TOK, NC, false> : gqa_mfma_kernel<QT, KV, false, TOK, NC, false>,
                  dim3(items), dim3(64), stream, ev, p, items);
  } else {
    auto kern = p.paged ? (p.balanced ? gqa_mfma_kernel<QT, KV, true, TOK, NC, true>
                                      : gqa_mfma_kernel<QT, KV, true, TOK, NC, false>)
                        : (p.balanced ? gqa_mfma_kernel<QT, KV, false, TOK, NC, true>
                                      : gqa_mfma_kernel<QT, KV, false, TOK, NC, false>);
    launch_kernel(kern, dim3(items), dim3(64), stream, ev, p, items);
  }
  return hipGetLastError();
}

// A KV head's query rows fill MFMA columns: 16 per wave when there are at
// most 16 of them (16x16x32 MFMAs: half the softmax, score and output
// registers of the 32-column layout for the padding that remains), else 32.
template <int QT, int KV, bool TOK>
hipError_t launch_kv(const GqaLaunch& p, hipStream_t stream, const LaunchEvents* ev) {
  return p.rows_kv <= 16 ? launch_nc<QT, KV, TOK, 16>(p, stream, ev) : launch_nc<QT, KV, TOK, 32>(p, stream, ev);
}

template <int QT>
hipError_t launch_i8(const GqaLaunch& p, hipStream_t stream, const LaunchEvents* ev) {
  return p.aq_token ? launch_kv<QT, kI8, true>(p, stream, ev) : launch_kv<QT, kI8, false>(p, stream, ev);
}

}  // namespace

bool gqa_mfma_supported(int q_dtype, int kv_dtype, int head_dim) {
  if (head_dim != kD) return false;
  if (kv_dtype == kI8) return q_dtype == kF32 || q_dtype == kF16 || q_dtype == kBF16;
  return q_dtype == kv_dtype && (kv_dtype == kF16 || kv_dtype == kBF16);
}

hipError_t launch_gqa_mfma(const GqaLaunch& p, hipStream_t stream, const LaunchEvents* ev) {
  if (!gqa_mfma_supported(p.q_dtype, p.kv_dtype, p.head_dim)) return hipErrorInvalidValue;
  if (p.kv_dtype == kI8) {
    switch (p.q_dtype) {
      case kF32: return launch_i8<kF32>(p, stream, ev);
      case kF16: return launch_i8<kF16>(p, stream, ev);
      default: return launch_i8<kBF16>(p, stream, ev);
    }
  }
  if (p.aq_token) return hipErrorInvalidValue;
  return p.kv_dtype == kBF16 ? launch_kv<kBF16, kBF16, false>(p, stream, ev)
                             : launch_kv<kF16, kF16, false>(p, stream, ev);
}

}  // namespace ifa
