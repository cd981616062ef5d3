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
// split).  The waves take 16-token tiles of the split round robin.  Inside a
// wave, C = D/16 lanes share one token row (16 channels per lane, loaded as
// 16-byte chunks so that each load instruction reads whole 128-byte row
// segments), so a wave step covers 64/C tokens.  q for the GH heads stays in
// registers.  Per tile: QK^T (packed dot2 for f16/bf16), a C-lane DPP
// reduction, the tile max over the wave, one rescale of the running
// (max, sum, acc) if the max grew, then P V in fp32 FMAs.  The next tile's
// K/V rows are loaded while the current one is computed.  At the end the
// waves merge their (max, sum, acc) through LDS and the workgroup writes the
// normalised partial.
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
    return __uint_as_float(r[i][k]);
  } else if constexpr (KV == kBF16) {
    const uint32_t w = r[i][k >> 1];
    return (k & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
  } else if constexpr (KV == kF16) {
    const uint32_t w = r[i][k >> 1];
    half2_t h = __builtin_bit_cast(half2_t, w);
    return (k & 1) ? (float)h[1] : (float)h[0];
  } else {
    // (float)(byte) of the biased word maps to v_cvt_f32_ubyte{0..3}
    const uint32_t w = r[0][k >> 2] ^ 0x80808080u;
    return (float)((w >> (8 * (k & 3))) & 0xffu);
  }
}

template <int QT, int KV, int D, int GH, bool PAGED>
__global__ void __launch_bounds__(256) gqa_splitkv_kernel(const GqaLaunch a, int work_items) {
  constexpr int C = D / 16;           // lanes per token row
  constexpr int TOK = 64 / C;         // tokens per wave step
  constexpr int NSTEP = 16 / TOK;     // steps per 16-token tile
  constexpr int TILE = 16;
  constexpr int ESZ = KvInfo<KV>::esz;
  constexpr int E = 16 / ESZ;          // channels per 16-byte chunk
  constexpr int NCH = ESZ;             // chunks per lane
  constexpr bool DOT2 = (KV == kF16 || KV == kBF16);
  static_assert(D % 16 == 0 && C >= 4 && TOK * NSTEP == TILE, "head dim");

  const int w = xcd_remap(blockIdx.x, gridDim.x);
  if (w >= work_items) return;
  const int HG = a.group / GH;
  int rem = w;
  const int hg = rem % HG; rem /= HG;
  const int split = rem % a.n_split; rem /= a.n_split;
  const int g = rem % a.n_kv; rem /= a.n_kv;
  const int b = rem;

  int64_t L = a.seq_lens[b];
  L = L < 0 ? 0 : (L > a.s_cap ? a.s_cap : L);
  const int64_t per = split_chunk(L, a.n_split);
  const int64_t start = (int64_t)split * per;
  const int64_t end = (start + per < L) ? start + per : L;
  if (start >= end) return;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t = lane / C, c = lane % C;
  const int h0 = g * a.group + hg * GH;

  // ---- q (and the int8 K-side constant) for this lane's 16 channels ----
  // channel of element e: E * ((e / E) * C + c) + e % E
  float qf[DOT2 ? 1 : GH][DOT2 ? 1 : 16];
  uint32_t qp[DOT2 ? GH : 1][DOT2 ? 8 : 1];
  float kconst[GH];  // int8: sum_d q'_d (offset_d - 128), in score units
#pragma unroll
  for (int h = 0; h < GH; ++h) {
    const int64_t qrow = ((int64_t)b * a.n_q + h0 + h) * D;
    float part = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int d = E * ((e / E) * C + c) + e % E;
      float qv = DOT2 ? 0.f : load_as_f32<QT>(a.q, qrow + d);
      if constexpr (KV == kI8) {
        const float sc = a.aq_scale[(int64_t)g * D + d];
        const float off = a.aq_offset[(int64_t)g * D + d];
        qv *= sc;
        part = fmaf(qv, off - 128.f, part);
      }
      if constexpr (DOT2) {
        // q has the same dtype as K here: repack its raw bits
        const uint16_t* q16 = static_cast<const uint16_t*>(a.q);
        const uint32_t bits = q16[qrow + d];
        if (e & 1) qp[h][e >> 1] |= bits << 16; else qp[h][e >> 1] = bits;
      } else {
        qf[h][e] = qv;
      }
    }
    kconst[h] = (KV == kI8) ? group_sum<C>(part) : 0.f;
  }

  const char* kbase = static_cast<const char*>(a.k);
  const char* vbase = static_cast<const char*>(a.v);

  // row index (in token rows) of token j of this (b, g); j must be < end
  auto token_row = [&](int64_t j) -> int64_t {
    if constexpr (PAGED) {
      int blk = a.block_table[(int64_t)b * a.max_blocks + j / a.block_size];
      blk = blk < 0 ? 0 : (blk >= a.num_blocks ? a.num_blocks - 1 : blk);
      return ((int64_t)blk * a.n_kv + g) * a.block_size + j % a.block_size;
    } else {
      return ((int64_t)b * a.n_kv + g) * a.s_cap + j;
    }
  };

  auto load_tile = [&](int tile, u32x4 (&kr)[NSTEP][NCH], u32x4 (&vr)[NSTEP][NCH]) {
#pragma unroll
    for (int st = 0; st < NSTEP; ++st) {
      const int64_t j0 = start + (int64_t)tile * TILE + st * TOK;  // wave-uniform
      const bool valid = j0 + t < end;
      const int64_t row = token_row(j0 < end ? j0 : start) + t;
      const u32x4* kp = reinterpret_cast<const u32x4*>(kbase + row * (D * ESZ)) + c;
      const u32x4* vp = reinterpret_cast<const u32x4*>(vbase + row * (D * ESZ)) + c;
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        kr[st][i] = valid ? kp[i * C] : u32x4{0u, 0u, 0u, 0u};
        vr[st][i] = valid ? vp[i * C] : u32x4{0u, 0u, 0u, 0u};
      }
    }
  };

  float m2[GH], lsum[GH], acc[GH][16];
#pragma unroll
  for (int h = 0; h < GH; ++h) {
    m2[h] = kNegInf;
    lsum[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[h][e] = 0.f;
  }

  const int64_t n_tok = end - start;
  const int ntiles = (int)((n_tok + TILE - 1) / TILE);
  u32x4 kc[NSTEP][NCH], vc[NSTEP][NCH], kn[NSTEP][NCH], vn[NSTEP][NCH];
  int tile = wave;
  if (tile < ntiles) load_tile(tile, kc, vc);
  for (; tile < ntiles; tile += 4) {
    if (tile + 4 < ntiles) load_tile(tile + 4, kn, vn);

    float s[NSTEP][GH];
#pragma unroll
    for (int st = 0; st < NSTEP; ++st) {
      const int64_t j = start + (int64_t)tile * TILE + st * TOK + t;
      const bool valid = j < end;
#pragma unroll
      for (int h = 0; h < GH; ++h) {
        float part = 0.f;
        if constexpr (KV == kBF16) {
#pragma unroll
          for (int p = 0; p < 8; ++p) {
            const uint32_t kw = kc[st][p / 4][p % 4];
            part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, qp[h][p]),
                                                   __builtin_bit_cast(bf162_t, kw), part, false);
          }
        } else if constexpr (KV == kF16) {
#pragma unroll
          for (int p = 0; p < 8; ++p) {
            const uint32_t kw = kc[st][p / 4][p % 4];
            part = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, qp[h][p]),
                                          __builtin_bit_cast(half2_t, kw), part, false);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 16; ++e) part = fmaf(qf[h][e], elem_f32<KV>(kc[st], e), part);
        }
        const float dot = group_sum<C>(part);
        s[st][h] = valid ? (dot + kconst[h]) * a.scale_log2 : kNegInf;
      }
    }

#pragma unroll
    for (int h = 0; h < GH; ++h) {
      float mx = s[0][h];
#pragma unroll
      for (int st = 1; st < NSTEP; ++st) mx = fmaxf(mx, s[st][h]);
      mx = strided_max<C>(mx);
      const float mnew = fmaxf(m2[h], mx);
      if (mnew > m2[h]) {
        const float alpha = fast_exp2(m2[h] - mnew);
        lsum[h] *= alpha;
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[h][e] *= alpha;
        m2[h] = mnew;
      }
    }

#pragma unroll
    for (int st = 0; st < NSTEP; ++st) {
      float p[GH];
#pragma unroll
      for (int h = 0; h < GH; ++h) {
        p[h] = fast_exp2(s[st][h] - m2[h]);
        lsum[h] += p[h];
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float vf = elem_f32<KV>(vc[st], e);
#pragma unroll
        for (int h = 0; h < GH; ++h) acc[h][e] = fmaf(p[h], vf, acc[h][e]);
      }
    }

#pragma unroll
    for (int st = 0; st < NSTEP; ++st)
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        kc[st][i] = kn[st][i];
        vc[st][i] = vn[st][i];
      }
  }

  // ---- reduce over the token lanes of the wave ----
#pragma unroll
  for (int h = 0; h < GH; ++h) {
    lsum[h] = strided_sum<C>(lsum[h]);
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[h][e] = strided_sum<C>(acc[h][e]);
  }

  // ---- merge the 4 waves through LDS and write the partial ----
  __shared__ float sm_acc[4][GH][D];
  __shared__ float sm_m[4][GH];
  __shared__ float sm_l[4][GH];
  if (t == 0) {
#pragma unroll
    for (int h = 0; h < GH; ++h)
#pragma unroll
      for (int e = 0; e < 16; ++e) sm_acc[wave][h][E * ((e / E) * C + c) + e % E] = acc[h][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < GH; ++h) {
      sm_m[wave][h] = m2[h];
      sm_l[wave][h] = lsum[h];
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < GH * D; idx += 256) {
    const int h = idx / D, d = idx % D;
    float M = kNegInf;
#pragma unroll
    for (int wv = 0; wv < 4; ++wv) M = fmaxf(M, sm_m[wv][h]);
    float tot = 0.f, o = 0.f;
#pragma unroll
    for (int wv = 0; wv < 4; ++wv) {
      const float mw = sm_m[wv][h];
      if (mw != kNegInf) {
        const float f = fast_exp2(mw - M);
        tot = fmaf(sm_l[wv][h], f, tot);
        o = fmaf(sm_acc[wv][h][d], f, o);
      }
    }
    o = o / tot;
    if constexpr (KV == kI8) {
      const int64_t pi = ((int64_t)a.n_kv + g) * D + d;  // V parameters (index 1)
      o = a.aq_scale[pi] * (o - 128.f + a.aq_offset[pi]);
    }
    const int64_t row = (int64_t)b * a.n_q + h0 + h;
    a.ws_o[(row * a.n_split + split) * D + d] = o;
    if (d == 0) {
      a.ws_m[row * a.n_split + split] = M * kLn2;
      a.ws_l[row * a.n_split + split] = tot;
    }
  }
}

template <int QT, int KV, int D, int GH>
hipError_t launch_typed(const GqaLaunch& p, hipStream_t stream) {
  const int items = p.batch * p.n_kv * (p.group / GH) * p.n_split;
  if (items == 0) return hipSuccess;
  const int padded = (items + kNumXcd - 1) / kNumXcd * kNumXcd;
  if (p.paged)
    hipLaunchKernelGGL((gqa_splitkv_kernel<QT, KV, D, GH, true>), dim3(padded), dim3(256), 0, stream, p, items);
  else
    hipLaunchKernelGGL((gqa_splitkv_kernel<QT, KV, D, GH, false>), dim3(padded), dim3(256), 0, stream, p, items);
  return hipGetLastError();
}

template <int QT, int KV, int D>
hipError_t launch_gh(const GqaLaunch& p, hipStream_t stream) {
  switch (p.heads_per_wg) {
    case 1: return launch_typed<QT, KV, D, 1>(p, stream);
    case 2: return launch_typed<QT, KV, D, 2>(p, stream);
    case 4: return launch_typed<QT, KV, D, 4>(p, stream);
    case 8:
      if constexpr (KV == kF16 || KV == kBF16) return launch_typed<QT, KV, D, 8>(p, stream);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

template <int QT, int KV>
hipError_t launch_d(const GqaLaunch& p, hipStream_t stream) {
  switch (p.head_dim) {
    case 64: return launch_gh<QT, KV, 64>(p, stream);
    case 128: return launch_gh<QT, KV, 128>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int gqa_max_heads_per_wg(int kv_dtype, int head_dim) {
  (void)head_dim;
  return (kv_dtype == kF16 || kv_dtype == kBF16) ? 8 : 4;
}

bool gqa_supported(int q_dtype, int kv_dtype, int head_dim, int heads_per_wg) {
  if (head_dim != 64 && head_dim != 128) return false;
  if (heads_per_wg != 1 && heads_per_wg != 2 && heads_per_wg != 4 && heads_per_wg != 8) return false;
  if (heads_per_wg > gqa_max_heads_per_wg(kv_dtype, head_dim)) return false;
  if (kv_dtype == kI8) return q_dtype == kF32 || q_dtype == kF16 || q_dtype == kBF16;
  return q_dtype == kv_dtype && (kv_dtype == kF32 || kv_dtype == kF16 || kv_dtype == kBF16);
}

hipError_t launch_gqa_splitkv(const GqaLaunch& p, hipStream_t stream) {
  if (!gqa_supported(p.q_dtype, p.kv_dtype, p.head_dim, p.heads_per_wg)) return hipErrorInvalidValue;
  if (p.kv_dtype == kI8) {
    switch (p.q_dtype) {
      case kF32: return launch_d<kF32, kI8>(p, stream);
      case kF16: return launch_d<kF16, kI8>(p, stream);
      default: return launch_d<kBF16, kI8>(p, stream);
    }
  }
  switch (p.kv_dtype) {
    case kF32: return launch_d<kF32, kF32>(p, stream);
    case kF16: return launch_d<kF16, kF16>(p, stream);
    default: return launch_d<kBF16, kBF16>(p, stream);
  }
}

}  // namespace ifa
