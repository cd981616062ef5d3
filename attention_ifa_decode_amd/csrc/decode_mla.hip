// MLA-shaped split-KV decode on the matrix cores (gfx950).
//
// The absorbed multi-head latent attention decode of the MlaProlog pages
// (aclnnMlaPrologV3WeightNz: query (B, S, N, 512 + 64), one combined
// latent + rope cache row of 576 channels per token, V = the first 512
// channels of that row) computes, per batch b and query head h,
//   Softmax(scale * q_h K^T) V                (aclnnIncreFlashAttentionV3, "Function")
// over the paged cache (page attention layout (blocknum, 1, blocksize, 576)).
// All N query heads share the one KV head, so QK^T and PV are dense
// contractions with M = heads: this path runs them on MFMA
// (v_mfma_f32_32x32x16_bf16) and writes the split partial triples
// (aclnnRingAttentionUpdate, "功能说明") that the combine kernel merges.
//
// Work decomposition.  A workgroup takes a group of up to 128 heads (wave w
// owns 32) over one or more pieces (sequence, token range):
//   - per-sequence split: one piece, split s of one sequence;
//   - balanced split: the batch's 32-token tiles, sequence after sequence,
//     cut into equal runs, one per workgroup, so that every compute unit
//     gets the same number of tiles whatever the length mix; a run yields a
//     piece for each sequence it touches.
// A piece's tokens stream through LDS in tiles of 32 rows x 1152 bytes,
// fetched straight from HBM into a 4-deep ring (global_load_lds_dwordx4,
// issued by all waves, one barrier per tile).  Per tile and wave:
//   S^T (32 tokens x 32 heads) = K (32 x 576) . Q^T (576 x 32): 36 MFMAs, K
//       read from LDS (ds_read_b128), Q^T held in registers for the piece;
//   online softmax per head (each lane holds one head column), with a lazy
//       rescale that only moves the running reference when a score exceeds
//       it by 2^8;
//   O^T (512 x 32) += V^T (512 x 32 tokens) . P^T (32 tokens x 32): 32 MFMAs.
//       P^T comes straight from the S^T accumulator (rounded to bf16); V^T is
//       read from the same K rows with the transposing LDS read
//       ds_read_b64_tr_b16, so V costs neither HBM nor LDS space of its own.
// Rows of a tile sit in LDS with their 16-byte chunks XOR-swizzled
// (position = chunk ^ f(row), f(row) = (2 (row & 3) + ((row >> 2) & 1)) ^
// (2 ((row >> 3) & 1))) so that both the row-wise K reads and the column-wise
// V^T reads are free of bank conflicts, whether the LDS serves 16-byte reads
// in phases of 8 lanes over 32 banks or of 16 lanes over 64 banks.
#include "common.hpp"
#include "kernels.hpp"

namespace ifa {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) short s16x4_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4_t;

constexpr int kDqk = 576, kDv = 512;
constexpr int kRowBytes = kDqk * 2;             // 1152 bytes per cached token row
constexpr int kChunks = kRowBytes / 16;         // 72 chunks of 16 bytes
constexpr int kTile = 32;                       // tokens per tile
constexpr int kTileBytes = kTile * kRowBytes;   // 36 KB
constexpr int kTileLoads = kTile * kChunks / 64;  // 36 wave-wide 1-KB loads per tile
constexpr int kKSteps = kDqk / 16;              // 36 MFMA k-steps for S^T
constexpr int kMTiles = kDv / 32;               // 16 row tiles of O^T
constexpr float kRescale = 8.f;                 // log2 headroom of the lazy rescale
constexpr float kMrefInit = -1e30f;

// Swizzle of row t: the 16-byte chunk c of the row is stored at position
// c ^ swz(t) (only the low 3 bits change, so chunks stay inside their group
// of 8).  Rows t and t + 8 get different values, so 16 consecutive rows hit
// 16 different 16-byte bank groups.
__device__ __forceinline__ int swz(int t) { return (2 * (t & 3) + ((t >> 2) & 1)) ^ (2 * ((t >> 3) & 1)); }

// Direct HBM -> LDS load of 16 bytes per lane from a per-lane address; the
// 64 lanes' bytes land contiguously at LDS byte address `lds` (+16 per lane).
// Issued from asm so that the compiler neither tracks it nor guards LDS
// reads against it; the ring is ordered with explicit vmcnt waits.
__device__ __forceinline__ void dma16_lane(const void* src, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, off offset:0 nt" ::"v"(src), "{m0}"(lds) : "memory");
}

// Same, from a wave-uniform base plus a 32-bit per-lane byte offset.
__device__ __forceinline__ void dma16_off(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, %1 offset:0 nt" ::"v"(voff), "s"(base), "{m0}"(lds) : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmem() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Make the compiler complete the loads behind `x` here rather than at its
// first use inside the streaming loop (where the wait would drain the ring).
template <typename T>
__device__ __forceinline__ void settle(const T& x) {
  asm volatile("" ::"v"(x));
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

__device__ __forceinline__ bf16x8_t lds_read_b128(uint32_t addr) {
  return *(const __attribute__((address_space(3))) bf16x8_t*)(uintptr_t)addr;
}

__device__ __forceinline__ f32x4_t lds_read_f32x4(uint32_t addr) {
  return *(const __attribute__((address_space(3))) f32x4_t*)(uintptr_t)addr;
}

__device__ __forceinline__ void lds_write_f32x4(uint32_t addr, f32x4_t v) {
  *(__attribute__((address_space(3))) f32x4_t*)(uintptr_t)addr = v;
}

__device__ __forceinline__ s16x4_t lds_read_tr16(uint32_t addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)(uintptr_t)addr);
}

// Multiply the 16 accumulator registers of one MFMA tile by `s` in place.
// Written as an accumulator-register read / multiply / write so that the
// tile stays in AGPRs: a plain VALU multiply would make the register
// allocator keep all 256 accumulator registers in VGPRs and spill.
__device__ __forceinline__ void scale_acc(f32x16_t& v, float s) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    float x = v[r];
    float tmp;
    asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                 : "+a"(x), "=&v"(tmp)
                 : "v"(s));
    v[r] = x;
  }
}

template <int NW>
struct MlaShape {
  static constexpr int LOADS_W = kTileLoads / NW;  // DMA instructions per wave per tile
  // tiles in flight, bounded by LDS (4 x 36 KB) and by the 6-bit vmcnt
  static constexpr int STAGES = (1 + 63 / LOADS_W) < 4 ? (1 + 63 / LOADS_W) : 4;
  static_assert(kTileLoads % NW == 0, "waves");
};

// OFF32: the whole cache lies within 4 GiB of its base (rows < 2^24), so a
// row's address is the base plus a 32-bit offset (24-bit multiplies).
template <int NW, bool PAGED, bool OFF32>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
mla_splitkv_kernel(const MlaLaunch a) {
  using S = MlaShape<NW>;
  constexpr int STAGES = S::STAGES, LOADS_W = S::LOADS_W;
  __shared__ __attribute__((aligned(16))) char ring[STAGES * kTileBytes];
  __shared__ int sm_blk[kMlaMaxTableSlice];
  // per-lane byte offsets of this wave's loads within a contiguous tile
  __shared__ uint32_t sm_loff[NW][LOADS_W][64];
  // balanced split: cost of the sequences before b (exclusive prefix), and
  // the tokens in each sequence's last tile
  __shared__ int sm_pref[kLongestFirstMaxBatch + 1];
  __shared__ uint8_t sm_rem[kLongestFirstMaxBatch];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = lane >> 5;  // which half of the MFMA k-range this lane feeds

  const char* kv = static_cast<const char*>(a.kv);
  const uint32_t ring_lds = lds_addr(ring);

  // A tile that holds 32 valid tokens of one cache block (or of the
  // contiguous layout) is 36 contiguous KB: lane l of this wave's load i then
  // reads byte t * 1152 + 16 ((P % 72) ^ swz(t)) of it, P = 64 (wave + NW i) + l,
  // t = P / 72, the same for every such tile.  Those offsets are computed once
  // into LDS (each lane reads back only its own); a tile then costs one
  // block-id read and, per load, one LDS read.  Other tiles (straddling a
  // block boundary, or a piece's last) take plan_tile / issue_loads.
  if constexpr (OFF32) {
#pragma unroll
    for (int i = 0; i < LOADS_W; ++i) {
      const int P = 64 * (wave + NW * i) + lane;
      const int t = P / kChunks;
      sm_loff[wave][i][lane] = (uint32_t)(t * kRowBytes + 16 * ((P - kChunks * t) ^ swz(t)));
    }
  }

  // ---- work: the pieces (sequence, token range) this workgroup reduces ----
  // Per-sequence split: one piece, split `split` of the sequence of rank
  // `rank` (longest sequences first).  Balanced split: run `run` of the
  // batch's tiles, which may cover the end of one sequence, whole short
  // ones and the start of another; one piece per sequence it touches.
  const int HGM = a.n_q / (32 * NW);
  int id = blockIdx.x;
  // Workgroups go to the 8 XCDs round-robin (workgroup i to XCD i % 8), each
  // with its own L2.  In the balanced split, XCD x takes the consecutive ids
  // x G/8 .. (x + 1) G/8 - 1, so the runs of one sequence (which read the
  // same Q rows) and the head groups of one run (which read the same KV
  // tiles) mostly share an L2.
  if (a.balanced && (gridDim.x & 7) == 0) id = (id & 7) * (int)(gridDim.x >> 3) + (id >> 3);
  const int hg = id % HGM;
  id /= HGM;
  int b = 0, L = 0, start = 0, end = 0;
  int64_t pbase = 0;  // partial of head `head`: index pbase + head * pstride
  int pstride = 1;
  int run = 0, nrun = 0, tcur = 0, trun_end = 0, ttotal = 0;  // balanced split, in cost units
  if (!a.balanced) {
    const int split = id % a.n_split;
    const int rank = id / a.n_split;
    b = rank;
    if (a.longest_first) {
      // the ranking keys use the ring, which no load reaches before the
      // piece's first barrier
      const BatchPick pick = batch_of_rank(rank, a.seq_lens, a.batch, a.s_cap,
                                           reinterpret_cast<uint32_t*>(ring) + wave * kLongestFirstMaxBatch);
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
    pbase = (int64_t)b * a.n_q * a.n_split + split;
    pstride = a.n_split;
  } else {
    // Cost of a sequence: its tiles plus kMlaPieceCost for the start of a
    // piece on it (Q, block slice, the ring's first tiles and the partial's
    // store, measured at about 7 tiles); none for an empty one.  sm_pref[b]
    // = cost of sequences 0 .. b-1 (wave 0, 64 sequences per step).
    if (wave == 0) {
      int carry = 0;
      for (int c0 = 0; c0 < a.batch; c0 += 64) {
        const int bb = c0 + lane;
        int t = 0;
        if (bb < a.batch) {
          const int64_t L64 = a.seq_lens[bb];
          const int Lb = (int)(L64 < 0 ? 0 : (L64 > a.s_cap ? a.s_cap : L64));
          t = (Lb + kTile - 1) / kTile;
          sm_rem[bb] = (uint8_t)(t > 0 ? Lb - kTile * (t - 1) : 0);
          if (t > 0) t += kMlaPieceCost;
        }
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
          const int y = __shfl_up(t, d);
          if (lane >= d) t += y;
        }
        if (bb < a.batch) sm_pref[bb + 1] = carry + t;
        carry += __shfl(t, 63);
      }
      if (lane == 0) sm_pref[0] = 0;
    }
    __syncthreads();
    // (values read from LDS are uniform; readfirstlane keeps them in scalar registers)
    ttotal = __builtin_amdgcn_readfirstlane(sm_pref[a.batch]);
    // runs: min(n_split, total cost) of them, so that none is empty; run r
    // covers cost units [r V / R, (r + 1) V / R) (floors)
    nrun = min(a.n_split, ttotal);
    run = id;
    if (run >= nrun) return;
    tcur = (int)((int64_t)run * ttotal / nrun);
    trun_end = (int)((int64_t)(run + 1) * ttotal / nrun);
    // the sequence holding unit tcur: sm_pref[lo] <= tcur < sm_pref[hi]
    int lo = 0, hi = a.batch;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (__builtin_amdgcn_readfirstlane(sm_pref[mid]) <= tcur) lo = mid;
      else hi = mid;
    }
    b = lo;
  }

  for (;;) {
    if (a.balanced) {
      // sequence b spans units [pb, pe): kMlaPieceCost units for its start,
      // then one per tile from z on.  The run's units [tcur, trun_end) hold
      // its tiles [max(tcur, z), min(trun_end, pe)) - z; none when the run
      // ends inside the start units (the next run takes the sequence).
      const int pb = __builtin_amdgcn_readfirstlane(sm_pref[b]);
      const int pe = __builtin_amdgcn_readfirstlane(sm_pref[b + 1]);
      const int z = pb + kMlaPieceCost;
      if (trun_end <= z) break;
      const int first = max(tcur, z);
      L = (pe - z - 1) * kTile + (int)__builtin_amdgcn_readfirstlane(sm_rem[b]);
      start = (first - z) * kTile;
      end = min(L, (min(trun_end, pe) - z) * kTile);
      pbase = (int64_t)(run + b) * a.n_q;
      pstride = 1;
      if (first == z && hg == 0 && threadIdx.x == 0) {
        // the runs that take sequence b are run .. the one holding its last unit
        const int rlast = (int)(((int64_t)pe * nrun - 1) / ttotal);
        a.seg_desc[b] = make_int2(run + b, rlast - run + 1);
      }
    }
    const int ntiles = (end - start + kTile - 1) / kTile;
    __syncthreads();  // every wave is done with the previous piece's ring and block slice (or the ranking keys)

    // ---- block-table slice of the split, staged in LDS ----
    const int blk0 = PAGED ? start / a.block_size : 0;
    const int nblk = PAGED ? (end - 1) / a.block_size - blk0 + 1 : 0;  // <= kMlaMaxTableSlice (host check)
    if constexpr (PAGED) {
      const int32_t* bt = a.block_table + (int64_t)b * a.max_blocks + blk0;
      for (int i = threadIdx.x; i < nblk; i += NW * 64) {
        int v = bt[i];
        sm_blk[i] = v < 0 ? 0 : (v >= a.num_blocks ? a.num_blocks - 1 : v);
      }
    }
    __syncthreads();  // the block slice is in

    // Queue the direct-to-LDS loads of tile j (this wave's share) into a ring
    // slot.  LDS chunk position P of the tile holds row t = P / 72, chunk
    // (P % 72) ^ swz(t) of that row; rows past the split's end repeat its last
    // row.  plan_tile reads the ids of the (at most 3) cache blocks the tile's
    // 32 tokens lie in and, per lane, the byte offset of one tile row;
    // issue_loads then queues loads [i0, i0 + n) of this wave.
    struct TilePlan {
      int tstart;
      uint32_t dst, tok0, adj0, adj1, adj2;
      uint32_t rowoff;  // OFF32: lane r holds the byte offset of tile row r % 32
    };
    auto plan_tile = [&](int j, int slot) -> TilePlan {
      TilePlan tp;
      tp.tstart = start + kTile * j;
      tp.dst = ring_lds + slot * kTileBytes;
      tp.tok0 = tp.adj0 = tp.adj1 = tp.adj2 = 0;
      if constexpr (PAGED) {
        // token tok sits in block adj_sel at slot u - sel * block_size,
        // u = tok - tok0, sel = u / block_size (at most 3 blocks per tile)
        const uint32_t bi0 = fast_div((uint32_t)tp.tstart, a.bs_magic, a.bs_shift);
        const int k0 = (int)bi0 - blk0;
        tp.tok0 = bi0 * (uint32_t)a.block_size;
        tp.adj0 = (uint32_t)__builtin_amdgcn_readfirstlane(sm_blk[k0]);
        tp.adj1 = (uint32_t)__builtin_amdgcn_readfirstlane(sm_blk[min(k0 + 1, nblk - 1)]);
        tp.adj2 = (uint32_t)__builtin_amdgcn_readfirstlane(sm_blk[min(k0 + 2, nblk - 1)]);
      } else {
        tp.adj0 = (uint32_t)b * (uint32_t)a.s_cap;  // row of token 0 of the sequence
      }
      tp.rowoff = 0;
      if constexpr (OFF32) {
        const uint32_t u = (uint32_t)min(tp.tstart + (lane & 31), end - 1) - tp.tok0;
        uint32_t row = tp.adj0 + u;
        if constexpr (PAGED) {
          const uint32_t bs = (uint32_t)a.block_size;
          row = u >= 2 * bs ? tp.adj2 * bs + (u - 2 * bs) : (u >= bs ? tp.adj1 * bs + (u - bs) : tp.adj0 * bs + u);
        }
        tp.rowoff = __umul24(row, (uint32_t)kRowBytes);
      }
      return tp;
    };
    auto issue_loads = [&](const TilePlan tp, int i0, int n) {
#pragma unroll
      for (int i = i0; i < i0 + n; ++i) {
        const int ins = wave + NW * i;
        if constexpr (OFF32) {
          // the instruction's 64 chunks are chunks lane + k1 of tile row t0 and,
          // from lane 72 - k1 on, chunks lane + k1 - 72 of row t0 + 1
          const int t0 = (64 * ins) / kChunks;
          const int k1 = 64 * ins - kChunks * t0;
          const uint32_t r0 = __builtin_amdgcn_readlane(tp.rowoff, t0);
          const uint32_t r1 = __builtin_amdgcn_readlane(tp.rowoff, min(t0 + 1, kTile - 1));
          const bool second = lane >= kChunks - k1;
          const int pin = lane + k1 - (second ? kChunks : 0);
          const int sw = second ? swz(t0 + 1) : swz(t0);
          dma16_off(kv, (second ? r1 : r0) + 16u * (uint32_t)(pin ^ sw), tp.dst + 1024 * ins);
        } else {
          const int P = 64 * ins + lane;
          const int t = P / kChunks;
          const int c = (P - kChunks * t) ^ swz(t);
          const int tok = min(tp.tstart + t, end - 1);
          uint64_t row;
          if constexpr (PAGED) {
            const uint32_t bs = (uint32_t)a.block_size;
            const uint32_t u = (uint32_t)tok - tp.tok0;
            row = u >= 2 * bs ? (uint64_t)tp.adj2 * bs + (u - 2 * bs)
                              : (u >= bs ? (uint64_t)tp.adj1 * bs + (u - bs) : (uint64_t)tp.adj0 * bs + u);
          } else {
            row = (uint64_t)tp.adj0 + (uint32_t)tok;
          }
          dma16_lane(kv + row * kRowBytes + 16 * c, tp.dst + 1024 * ins);
        }
      }
    };

    auto queue_tile = [&](int j, int slot) {
      if constexpr (OFF32) {
        const int tstart = start + kTile * j;
        bool whole = tstart + kTile <= end;
        uint32_t row0 = 0;
        if constexpr (PAGED) {
          const uint32_t bi = fast_div((uint32_t)tstart, a.bs_magic, a.bs_shift);
          const uint32_t u = (uint32_t)tstart - bi * (uint32_t)a.block_size;
          whole = whole && u + kTile <= (uint32_t)a.block_size;
          if (whole)
            row0 = (uint32_t)__builtin_amdgcn_readfirstlane(sm_blk[(int)bi - blk0]) * (uint32_t)a.block_size + u;
        } else {
          row0 = (uint32_t)b * (uint32_t)a.s_cap + (uint32_t)tstart;
        }
        if (whole) {
          const char* base = kv + (uint64_t)row0 * kRowBytes;
          const uint32_t dst = ring_lds + slot * kTileBytes;
          uint32_t off[LOADS_W];
#pragma unroll
          for (int i = 0; i < LOADS_W; ++i) off[i] = sm_loff[wave][i][lane];
#pragma unroll
          for (int i = 0; i < LOADS_W; ++i) dma16_off(base, off[i], dst + 1024 * (wave + NW * i));
          return;
        }
      }
      issue_loads(plan_tile(j, slot), 0, LOADS_W);
    };

    // ---- Q^T operand: this wave's 32 heads, 8 channels per lane per k-step ----
    // The row address comes from a lane index laundered per piece: a hoisted
    // copy would be spilled, and reloading it waits for every older load,
    // tile 0's included, before Q's loads can go out.
    int qlane = lane;
    asm volatile("" : "+v"(qlane));
    const int head = hg * (32 * NW) + wave * 32 + (qlane & 31);
    const int64_t qoff = ((int64_t)b * a.n_q + head) * kRowBytes + 16 * (qlane >> 5);
    const bf16x8_t* qrow = reinterpret_cast<const bf16x8_t*>(static_cast<const char*>(a.q) + qoff);
    // Tile 0 is queued first so that its loads and Q's are in flight
    // together; the wait for Q (older loads complete first) then covers
    // tile 0, which the first step needs anyway.
    queue_tile(0, 0);
    bf16x8_t qreg[kKSteps];
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) qreg[ks] = qrow[2 * ks];
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) settle(qreg[ks]);

#pragma unroll
    for (int s = 1; s < STAGES - 1; ++s)
      if (s < ntiles) queue_tile(s, s);

    // ---- per-lane LDS offsets (relative to a tile's slot) ----
    // S^T A operand: token t = lane % 32, chunk 2 ks + h at position
    // 8 (ks / 4) + ((2 (ks % 4) + h) ^ swz(t)).
    uint32_t offS[4];
    {
      const int t = lane & 31;
#pragma unroll
      for (int j = 0; j < 4; ++j) offS[j] = t * kRowBytes + 16 * ((2 * j + h) ^ swz(t));
    }
    // V^T A operand through the transposing read.  In each 16-lane group g,
    // source lane s reads 4 channels (8 bytes) of row kbase + s / 4 at column
    // nbase + 4 (s % 4); the read hands lane i of the group the 4 tokens
    // kbase..kbase+3 of column nbase + i.  MFMA row (V channel) = lane % 32,
    // i.e. nbase = 32 mt + 16 (g % 2); the k-slots of lane half h are the
    // tokens 4h..4h+3 (first read) and 8+4h..8+4h+3 (second read) of each
    // 16-token k-step, which is the token order of the S^T accumulator rows
    // that feed P^T.
    uint32_t offV[2][2];  // [odd mt][second read, 8 rows further]
    {
      const int s = lane & 15, g = lane >> 4;
      const int r = s >> 2, q = s & 3;
#pragma unroll
      for (int rd = 0; rd < 2; ++rd) {
        const int t = 8 * rd + 4 * (g >> 1) + r;  // row within the 16-token k-step
#pragma unroll
        for (int odd = 0; odd < 2; ++odd) {
          const int x = 4 * odd + 2 * (g & 1) + (q >> 1);  // chunk within the 8-chunk group
          offV[odd][rd] = t * kRowBytes + 16 * (x ^ swz(t)) + 8 * (q & 1);
        }
      }
    }

    // lsum: sum of the fp32 weights (the partial's softmax_sum, hence lse);
    // lsum_r: sum of the bf16-rounded weights that enter PV (normalises out)
    float mref = kMrefInit, mtrue = kNegInf, lsum = 0.f, lsum_r = 0.f;
    f32x16_t acc[kMTiles];
#pragma unroll
    for (int mt = 0; mt < kMTiles; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mt][r] = 0.f;

    for (int i = 0; i < ntiles; ++i) {
      // tile i has landed once at most the loads of the tiles queued after it
      // are in flight (vmcnt retires in order)
      const int after = min(STAGES - 2, ntiles - 1 - i);
      if constexpr (STAGES >= 4) {
        if (after >= 2) wait_vmem<2 * LOADS_W>();
        else if (after == 1) wait_vmem<LOADS_W>();
        else wait_vmem<0>();
      } else if constexpr (STAGES == 3) {
        if (after >= 1) wait_vmem<LOADS_W>();
        else wait_vmem<0>();
      } else {
        wait_vmem<0>();
      }
      __syncthreads();  // every wave's share of tile i is in; tile i-1 is consumed
      const uint32_t slot = ring_lds + (i % STAGES) * kTileBytes;
      const int tstart = start + kTile * i;

      // ---- S^T = K . Q^T (one accumulator: a second one would leave no
      // registers for reading K ahead of the MFMAs) ----
      f32x16_t sacc;
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
      uint32_t bS[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) bS[j] = slot + offS[j];
      // K operands are read one group of 4 k-steps ahead of their MFMAs; the
      // scheduling fences keep the compiler from pulling each read down next to
      // its MFMA (which would expose the full LDS latency at every step)
      bf16x8_t kbuf[2][4];
#pragma unroll
      for (int j = 0; j < 4; ++j) kbuf[0][j] = lds_read_b128(bS[j]);
#pragma unroll
      for (int grp = 0; grp < kKSteps / 4; ++grp) {
        if (grp + 1 < kKSteps / 4) {
#pragma unroll
          for (int j = 0; j < 4; ++j) kbuf[(grp + 1) & 1][j] = lds_read_b128(bS[j] + 128 * (grp + 1));
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kbuf[grp & 1][j], qreg[4 * grp + j], sacc, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }

      // ---- online softmax over this lane's head (column) ----
      // accumulator register r holds token 8 (r / 4) + 4 h + r % 4 of the tile
      float sv[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) sv[r] = sacc[r] * a.scale_log2;
      if (tstart + kTile > end) {  // the split's last tile: tokens past its end weigh 0
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (tstart + 8 * (r >> 2) + 4 * h + (r & 3) >= end) sv[r] = kNegInf;
      }
      float smax = kNegInf;
#pragma unroll
      for (int r = 0; r < 16; ++r) smax = fmaxf(smax, sv[r]);
      smax = xor32_max(smax);  // the other 16 tokens of the column sit in lane ^ 32
      mtrue = fmaxf(mtrue, smax);
      if (__builtin_amdgcn_ballot_w64(smax > mref + kRescale)) {  // rare after the first tile
        const float mnew = smax > mref + kRescale ? smax : mref;
        const float alpha = fast_exp2(mref - mnew);  // 0 on the first tile
        lsum *= alpha;
        lsum_r *= alpha;
#pragma unroll
        for (int mt = 0; mt < kMTiles; ++mt) scale_acc(acc[mt], alpha);
        mref = mnew;
      }
      // P^T operand: k-slot j of lane half h is accumulator register j (k-step 0)
      // or 8 + j (k-step 1)
      bf16x8_t pb[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pf = fast_exp2(sv[r] - mref);  // <= 2^8; 0 past the end
        pb[r >> 3][r & 7] = (__bf16)pf;
        lsum += pf;
      }
      const bf162_t ones = {(__bf16)1.f, (__bf16)1.f};
#pragma unroll
      for (int r = 0; r < 16; r += 2)
        lsum_r = __builtin_amdgcn_fdot2_f32_bf16(bf162_t{pb[r >> 3][r & 7], pb[r >> 3][(r & 7) + 1]}, ones, lsum_r,
                                                 false);

      // keep the softmax out of the PV schedule: interleaving it would lengthen
      // register live ranges and starve the V^T read-ahead
      __builtin_amdgcn_sched_barrier(0);

      // Tile i + STAGES - 1 goes into the slot of tile i - 1, free since the
      // barrier.  Queued here rather than right after it, its loads do not
      // hold up the first QK^T MFMAs; PV waits on LDS reads anyway.
      if (i + STAGES - 1 < ntiles) queue_tile(i + STAGES - 1, (i + STAGES - 1) % STAGES);
      __builtin_amdgcn_sched_barrier(0);

      // ---- O^T += V^T . P^T (MFMA n: k-step n / 16, row tile n % 16) ----
      const uint32_t bV[2][2] = {{slot + offV[0][0], slot + offV[0][1]}, {slot + offV[1][0], slot + offV[1][1]}};
      auto vread = [&](int n) -> bf16x8_t {
        const int kk = n / kMTiles, mt = n % kMTiles;
        const uint32_t imm = kRowBytes * 16 * kk + 128 * (mt >> 1);
        const s16x4_t lo = lds_read_tr16(bV[mt & 1][0] + imm);
        const s16x4_t hi = lds_read_tr16(bV[mt & 1][1] + imm);
        return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      };
      // V^T operands are read one group of 4 MFMAs ahead (scheduling fences as
      // in QK^T)
      bf16x8_t vbuf[2][4];
#pragma unroll
      for (int j = 0; j < 4; ++j) vbuf[0][j] = vread(j);
#pragma unroll
      for (int grp = 0; grp < 2 * kMTiles / 4; ++grp) {
        if (grp + 1 < 2 * kMTiles / 4) {
#pragma unroll
          for (int j = 0; j < 4; ++j) vbuf[(grp + 1) & 1][j] = vread(4 * (grp + 1) + j);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int n = 4 * grp + j;
          acc[n % kMTiles] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(vbuf[grp & 1][j], pb[n / kMTiles], acc[n % kMTiles], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // ---- partial triple: normalised out, true max, sum relative to it ----
    const float ltot = xor32_sum(lsum);
    const float inv = 1.f / xor32_sum(lsum_r);
    const int64_t pidx = pbase + (int64_t)head * pstride;
    // O^T leaves through LDS, 128 channels at a time: lane (head, h) holds
    // 4 consecutive channels of its head per accumulator quad, so direct
    // stores would write 8-byte (fp16) pieces of 32 rows; read back
    // row-wise, each store writes 256 contiguous bytes of each of two heads'
    // rows.  The partial outputs are fp16 (max and sum stay fp32): a
    // normalised partial is a convex combination of V rows, within fp16's
    // range as long as V is.  The wave uses
    // half of a ring slot that no wave reads any more (every slot but the
    // last tile's is free once the wave has left the loop; the next piece's
    // first barrier orders the reuse).  Rows are padded to 528 bytes, which
    // keeps both the writes and the reads free of bank conflicts.
    {
      constexpr int kORow = 128 * 4 + 16;
      const int last = (ntiles - 1) % STAGES;
      const uint32_t obuf = ring_lds + ((last + 1 + (wave >> 1)) % STAGES) * kTileBytes + (wave & 1) * 32 * kORow;
      const int hl = lane & 31;
      // this lane's first row (head h of the wave) at channel 4 hl; its later
      // rows follow every two heads.  The address advances by one stride per
      // store: left to itself the compiler precomputed the 16 row addresses
      // (64-bit products) once, held them across the 4 rounds and spilled
      // them, and each store then waited for its reload.
      _Float16* const lane_row = a.ws_o + (pbase + (int64_t)(head - hl + h) * pstride) * kDv + 4 * hl;
      const int64_t row_step = 2 * (int64_t)pstride * kDv;
#pragma unroll
      for (int c = 0; c < kMTiles / 4; ++c) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            f32x4_t v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = acc[4 * c + j][4 * q + e] * inv;
            lds_write_f32x4(obuf + hl * kORow + 4 * (32 * j + 8 * q + 4 * h), v);
          }
        int64_t off = 128 * c;
        asm volatile("" : "+v"(off));  // per round, not hoisted (an offset: the pointer stays global)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = 2 * i + h;  // row (head of the wave) this lane stores
          const f32x4_t v = lds_read_f32x4(obuf + r * kORow + 16 * hl);
          // rounded to fp16 (nearest even): 256 contiguous bytes per row
          const f16x4_t w = {(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
          *reinterpret_cast<f16x4_t*>(lane_row + off) = w;
          off += row_step;
        }
      }
    }
    if (h == 0) {
      a.ws_m[pidx] = mtrue * kLn2;
      a.ws_l[pidx] = ltot * fast_exp2(mref - mtrue);
    }

    // next piece: the next sequence with tiles, while the run lasts
    if (!a.balanced) break;
    tcur = min(trun_end, (int)__builtin_amdgcn_readfirstlane(sm_pref[b + 1]));
    if (tcur >= trun_end) break;
    do {
      ++b;  // stays below batch: units remain after tcur
    } while (__builtin_amdgcn_readfirstlane(sm_pref[b + 1]) == tcur);
  }
}

template <int NW>
hipError_t launch_nw(const MlaLaunch& p, hipStream_t stream, const LaunchEvents* ev) {
  // per-sequence split: (sequence, split, head group); balanced: (run, head group)
  const int items = (p.balanced ? 1 : p.batch) * p.n_split * (p.n_q / (32 * NW));
  if (items == 0) return hipSuccess;
  const uint64_t rows = p.paged ? (uint64_t)p.num_blocks * (uint64_t)p.block_size : (uint64_t)p.batch * (uint64_t)p.s_cap;
  const bool off32 = rows * kRowBytes < (1ull << 32);
  auto kern = p.paged ? (off32 ? mla_splitkv_kernel<NW, true, true> : mla_splitkv_kernel<NW, true, false>)
                      : (off32 ? mla_splitkv_kernel<NW, false, true> : mla_splitkv_kernel<NW, false, false>);
  launch_kernel(kern, dim3(items), dim3(NW * 64), stream, ev, p);
  return hipGetLastError();
}

}  // namespace

bool mla_supported(int n_q) { return n_q >= 32 && n_q % 32 == 0; }

hipError_t launch_mla_splitkv(const MlaLaunch& p, hipStream_t stream, const LaunchEvents* ev) {
  if (p.qk_dim != kDqk || p.v_dim != kDv || !mla_supported(p.n_q)) return hipErrorInvalidValue;
  if (p.n_q % 128 == 0) return launch_nw<4>(p, stream, ev);
  if (p.n_q % 64 == 0) return launch_nw<2>(p, stream, ev);
  return launch_nw<1>(p, stream, ev);
}

}  // namespace ifa
