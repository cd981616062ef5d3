// Device helpers shared by the decode, combine and update kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.hpp"

namespace ifa {

enum DType : int { kF32 = 0, kF16 = 1, kBF16 = 2, kI8 = 3 };

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

typedef __attribute__((ext_vector_type(2))) _Float16 half2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf162_t;
typedef __attribute__((ext_vector_type(4))) float float4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

// Element i of a 4-dword vector, by value.  Always go through this before a
// __builtin_bit_cast: applied directly to a vector-element lvalue, the bit
// cast reads element 0 with the ROCm 7.2 clang (observed on gfx950 code).
__device__ __forceinline__ uint32_t word(const u32x4& v, int i) {
  const uint32_t w = v[i];
  return w;
}

// ---------------------------------------------------------------------------
// scalar conversions
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <int DT>
__device__ __forceinline__ float load_as_f32(const void* base, int64_t idx);

template <>
__device__ __forceinline__ float load_as_f32<kF32>(const void* base, int64_t idx) {
  return static_cast<const float*>(base)[idx];
}
template <>
__device__ __forceinline__ float load_as_f32<kF16>(const void* base, int64_t idx) {
  return (float)static_cast<const _Float16*>(base)[idx];
}
template <>
__device__ __forceinline__ float load_as_f32<kBF16>(const void* base, int64_t idx) {
  return bf16_bits_to_f32(static_cast<const uint16_t*>(base)[idx]);
}
template <>
__device__ __forceinline__ float load_as_f32<kI8>(const void* base, int64_t idx) {
  return (float)static_cast<const int8_t*>(base)[idx];
}

template <int DT>
__device__ __forceinline__ void store_from_f32(void* base, int64_t idx, float v);

template <>
__device__ __forceinline__ void store_from_f32<kF32>(void* base, int64_t idx, float v) {
  static_cast<float*>(base)[idx] = v;
}
template <>
__device__ __forceinline__ void store_from_f32<kF16>(void* base, int64_t idx, float v) {
  static_cast<_Float16*>(base)[idx] = (_Float16)v;  // v_cvt_f16_f32: round to nearest even
}
template <>
__device__ __forceinline__ void store_from_f32<kBF16>(void* base, int64_t idx, float v) {
  static_cast<uint16_t*>(base)[idx] = f32_to_bf16_bits(v);
}

// ---------------------------------------------------------------------------
// cross-lane reductions
// ---------------------------------------------------------------------------

// DPP controls (GFX9 encoding).
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowRor4 = 0x124;
constexpr int kDppRowRor8 = 0x128;

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Sum over aligned groups of N consecutive lanes (N in 1,2,4,8,16); every lane
// of the group receives the group sum.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += dpp_f32<kDppQuadXor1>(x);
  if constexpr (N >= 4) x += dpp_f32<kDppQuadXor2>(x);
  if constexpr (N >= 8) x += dpp_f32<kDppRowHalfMirror>(x);
  if constexpr (N >= 16) x += dpp_f32<kDppRowMirror>(x);
  return x;
}

// Cross-row exchanges (gfx950 v_permlane16/32_swap).  Called with the same
// value for both operands, the two results hold, at every lane, the value of
// that lane's row and of its partner row (rows of 16 lanes: partner = row^1
// for the 16-swap, row^2 for the 32-swap), so their sum / max is the
// all-reduce over lanes l and l^16 (l^32).
__device__ __forceinline__ float xor16_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor16_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// All-reduce over the lanes that differ only in lane-id bits log2(STRIDE)..5
// (STRIDE in 4, 8, 16, 32).  Inside a 16-lane row, rotations by 4 and 8 visit
// the four quads; rows are combined with the permlane swaps.
template <int STRIDE>
__device__ __forceinline__ float strided_sum(float x) {
  static_assert(STRIDE == 4 || STRIDE == 8 || STRIDE == 16 || STRIDE == 32, "stride");
  if constexpr (STRIDE <= 4) x += dpp_f32<kDppRowRor4>(x);
  if constexpr (STRIDE <= 8) x += dpp_f32<kDppRowRor8>(x);
  if constexpr (STRIDE <= 16) x = xor16_sum(x);
  return xor32_sum(x);
}

template <int STRIDE>
__device__ __forceinline__ float strided_max(float x) {
  static_assert(STRIDE == 4 || STRIDE == 8 || STRIDE == 16 || STRIDE == 32, "stride");
  if constexpr (STRIDE <= 4) x = fmaxf(x, dpp_f32<kDppRowRor4>(x));
  if constexpr (STRIDE <= 8) x = fmaxf(x, dpp_f32<kDppRowRor8>(x));
  if constexpr (STRIDE <= 16) x = xor16_max(x);
  return xor32_max(x);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// XCD-aware work mapping.  Consecutive workgroup ids are dispatched round
// robin over the 8 XCDs; this maps a linear id to a work index so that
// consecutive work indices sit on the same XCD (and so share its L2).
// `padded` is the grid size, a multiple of 8.
// ---------------------------------------------------------------------------
constexpr int kNumXcd = 8;

__device__ __forceinline__ int xcd_remap(int id, int padded) {
  const int per = padded / kNumXcd;
  return (id % kNumXcd) * per + id / kNumXcd;
}

// Load through the constant address space: with a wave-uniform index this
// becomes a scalar load (s_load).  Scalar loads travel through the scalar
// cache, so under load they do not queue behind the CU's in-flight vector
// loads (measured while the decode kernel streams: about 0.2 us against
// 1.7 us), and they are tracked by lgkmcnt, not vmcnt.
template <typename T>
__device__ __forceinline__ T ld_uniform(const T* p, int64_t i) {
  return ((const __attribute__((address_space(4))) T*)p)[i];
}

// n (<= 64) consecutive 32-bit values from p through scalar loads, value k
// into lane k of the result (other lanes: `fill`).  Whole groups of 16 become
// one 64-byte scalar load each.
__device__ __forceinline__ int lanes_from_scalar_loads(const int* p, int n, int fill) {
  int v = fill;
  for (int k0 = 0; k0 < n; k0 += 16) {
    int x[16];
    if (k0 + 16 <= n) {
#pragma unroll
      for (int k = 0; k < 16; ++k) x[k] = ld_uniform(p, k0 + k);
    } else {
#pragma unroll
      for (int k = 0; k < 16; ++k) x[k] = k0 + k < n ? ld_uniform(p, k0 + k) : fill;
    }
    const int rel = (int)(threadIdx.x & 63) - k0;
#pragma unroll
    for (int k = 0; k < 16; ++k) v = rel == k ? x[k] : v;
  }
  return v;
}

// Longest-first order.  Sequences are ordered by descending clamped length
// (ties by batch index); dispatching long sequences first keeps the last
// workgroups short (longest-processing-time-first list scheduling).  Each
// sequence gets a unique 32-bit key, (min(len, 2^23 - 1) + 1) * 256 + 255 - i,
// so its rank is the number of larger keys: the keys go to LDS
// (kLongestFirstMaxBatch entries) and every lane counts against all of them
// through broadcast LDS reads.  Lengths beyond 2^23 tie in the key and are
// ordered by index.  Requires batch <= kLongestFirstMaxBatch.
constexpr int kRankChunks = kLongestFirstMaxBatch / 64;
static_assert(kLongestFirstMaxBatch <= 256, "8-bit index in the key");

// Key of sequence i with clamped length x (x < 0: padding, key 0, below
// every real key).
__device__ __forceinline__ uint32_t longest_first_key(int64_t x, int i) {
  return x < 0 ? 0u : (((uint32_t)(x < (1 << 23) - 1 ? x : (1 << 23) - 1) + 1u) << 8) | (uint32_t)(255 - i);
}

// r[c] = number of the nc * 64 keys in LDS that exceed key[c].
__device__ __forceinline__ void count_larger(const uint32_t* keys, int nc, const uint32_t (&key)[kRankChunks],
                                             int (&r)[kRankChunks]) {
  const uint4* k4 = reinterpret_cast<const uint4*>(keys);
#pragma unroll
  for (int c = 0; c < kRankChunks; ++c) r[c] = 0;
  for (int j = 0; j < nc * 16; ++j) {
    const uint4 q = k4[j];
#pragma unroll
    for (int c = 0; c < kRankChunks; ++c)
      r[c] += (int)(q.x > key[c]) + (int)(q.y > key[c]) + (int)(q.z > key[c]) + (int)(q.w > key[c]);
  }
}

// Ranks of all sequences, by one wave alone (no barrier) with `keys` as its
// own LDS: lane i of chunk c gets the clamped length of sequence 64 c + i in
// len[c] (-1 for padding) and its rank in rank[c].
__device__ inline void rank_lengths(const int64_t* lens, int batch, int64_t cap, uint32_t* keys,
                                    int (&len)[kRankChunks], int (&rank)[kRankChunks]) {
  const int lane = threadIdx.x & 63;
  const int nc = (batch + 63) >> 6;
  uint32_t key[kRankChunks];
#pragma unroll
  for (int c = 0; c < kRankChunks; ++c) {
    const int i = c * 64 + lane;
    int64_t x = -1;
    if (c < nc && i < batch) {
      x = lens[i];
      x = x < 0 ? 0 : (x > cap ? cap : x);
    }
    len[c] = (int)x;
    key[c] = longest_first_key(x, i);
    if (c < nc) keys[i] = key[c];
  }
  // LDS operations of one wave complete in order: the reads below see every
  // lane's write
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  count_larger(keys, nc, key, rank);
}

// The sequence that comes `rank`-th in longest-first order, and its clamped
// length.  Requires 0 <= rank < batch <= kLongestFirstMaxBatch.  The result
// is wave-uniform.
struct BatchPick {
  int b, len;
};

__device__ __forceinline__ BatchPick pick_rank(int rank, const int (&len)[kRankChunks], const int (&r)[kRankChunks]) {
  BatchPick p{rank, 0};  // replaced below: the ranks of the real lanes are a permutation of 0..batch-1
#pragma unroll
  for (int c = 0; c < kRankChunks; ++c) {
    const uint64_t m = __builtin_amdgcn_ballot_w64(len[c] >= 0 && r[c] == rank);
    if (m) {
      const int k = __builtin_ctzll(m);
      p.b = c * 64 + k;
      p.len = __builtin_amdgcn_readlane(len[c], k);
    }
  }
  return p;
}

// One wave alone, no barrier: a vector load of the lengths.
__device__ inline BatchPick batch_of_rank(int rank, const int64_t* lens, int batch, int64_t cap, uint32_t* keys) {
  int len[kRankChunks], r[kRankChunks];
  rank_lengths(lens, batch, cap, keys, len, r);
  return pick_rank(rank, len, r);
}

}  // namespace ifa
