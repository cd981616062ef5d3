// Merge kernels (gfx950): the n-way combine of split partials with the
// learnable sink, and the pairwise RingAttentionUpdate; and the small
// planning kernel that ranks the sequences for the split-KV kernels.
//
// Both apply the update rule of aclnnRingAttentionUpdate ("功能说明"), in its
// sum-weighted form: with M the largest softmax_max, every partial i enters
// with weight w_i = softmax_sum_i * e^(softmax_max_i - M) (zero for an empty
// partial whose max is -inf), the merged sum is sum_i w_i and the merged
// output is sum_i w_i attn_out_i / sum_i w_i.  The combine also folds the
// learnable sink of aclnnFlashAttentionScoreV4 ("计算公式": the denominator
// gains e^(sink - m) and m = max(sink, max S)) in as one more partial with
// attn_out 0, max sink, sum 1, and writes lse = M + ln(sum) (the softmaxLse
// output of the FusedInferAttentionScore blog).
//
// Both kernels are memory-bound passes with one wave per row.  The combine
// issues every load of a row (partials, statistics, length) before waiting,
// so a row costs one memory round trip whatever its split count.
#include "common.hpp"
#include "kernels.hpp"

namespace ifa {
namespace {

constexpr int kRowsPerBlock = 4;
constexpr int kMaxSplitsPerRow = 256;

__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_f32<kDppQuadXor1>(x));
  x = fmaxf(x, dpp_f32<kDppQuadXor2>(x));
  x = fmaxf(x, dpp_f32<kDppRowHalfMirror>(x));
  x = fmaxf(x, dpp_f32<kDppRowMirror>(x));
  return xor32_max(xor16_max(x));
}

__device__ __forceinline__ float wave_sum(float x) { return xor32_sum(xor16_sum(group_sum<16>(x))); }

// Four consecutive outputs; one vector store when the output buffer is
// 16-byte aligned (then every row start is, VD being a multiple of 64).
template <int OT>
__device__ __forceinline__ void store4(void* out, int64_t idx, const float4& v) {
  if ((reinterpret_cast<uintptr_t>(out) & 15) != 0) {
    store_from_f32<OT>(out, idx, v.x), store_from_f32<OT>(out, idx + 1, v.y);
    store_from_f32<OT>(out, idx + 2, v.z), store_from_f32<OT>(out, idx + 3, v.w);
  } else if constexpr (OT == kF32) {
    *reinterpret_cast<float4*>(static_cast<float*>(out) + idx) = v;
  } else {
    uint16_t h[4];
    if constexpr (OT == kF16) {
      const _Float16 f[4] = {(_Float16)v.x, (_Float16)v.y, (_Float16)v.z, (_Float16)v.w};
      __builtin_memcpy(h, f, sizeof(h));
    } else {
      h[0] = f32_to_bf16_bits(v.x), h[1] = f32_to_bf16_bits(v.y);
      h[2] = f32_to_bf16_bits(v.z), h[3] = f32_to_bf16_bits(v.w);
    }
    uint2 p;
    p.x = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
    p.y = (uint32_t)h[2] | ((uint32_t)h[3] << 16);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + idx) = p;
  }
}

// One wave per (batch, head) row.  A row's partial outputs are n_split
// contiguous vectors of VD values, fp32 or (H, the MLA path) fp16; lanes
// read them in 16-byte units of E = 4 or 8 channels, so a load instruction
// covers PARTS = 64 / (VD/E) splits (4 at VD 64, 2 at 128, 1 at 512, where
// fp32 lanes hold two units).  All loads of a batch of splits are issued
// before the statistics are reduced, so a row costs one memory round trip
// rather than one per split.
template <int OT, int VD, bool H>
__global__ void __launch_bounds__(256) combine_kernel(const CombineLaunch a) {
  constexpr int kE = H ? 8 : 4;  // channels per 16-byte unit
  constexpr int kUnits = VD / kE;
  constexpr int kLanesPerSplit = kUnits < 64 ? kUnits : 64;
  constexpr int kParts = 64 / kLanesPerSplit;
  constexpr int kCols = kUnits / kLanesPerSplit;
  // 16-byte loads in flight per lane: 16 at VD 512 (64 registers of them, so
  // that the kernel stays under 104 VGPRs and five waves fit per SIMD: a
  // launch of up to 1280 four-row workgroups is then resident in one round),
  // 8 below; a row with more splits takes further batches
  constexpr int kSteps = kCols == 2 ? 8 : (kParts == 1 ? 16 : 8);
  constexpr int kBatch = kSteps * kParts;  // splits per batch of loads
  __shared__ float sm_m[kRowsPerBlock][kMaxSplitsPerRow];
  __shared__ float sm_w[kRowsPerBlock][kMaxSplitsPerRow];

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = blockIdx.x * kRowsPerBlock + wave;  // rows < 2^31 (checked at launch)
  if (row >= a.batch * a.n_q) return;  // uniform per wave; no block barrier below
  const int b = row / a.n_q, h = row - b * a.n_q;
  const int part = lane / kLanesPerSplit, col = lane % kLanesPerSplit;

  // Partial s of the row: vector o[s * ostep], statistics m[s * mstep],
  // l[s * mstep]; slots [0, nload) lie in the workspace, of which the first
  // nvalid were written by this call.  In the per-sequence layout every load
  // of the row is issued before the length arrives; the balanced layout
  // reads the sequence's slot range first.
  int64_t L64 = a.seq_lens[b / a.q_seq];
  const int L = (int)(L64 < 0 ? 0 : (L64 > a.s_cap ? a.s_cap : L64));
  const uint4* o;
  const float *m, *l;
  const char* const wo = static_cast<const char*>(a.ws_o);
  constexpr int64_t kRowBytes = (int64_t)VD * (H ? 2 : 4);
  int ostep, mstep, nload, nvalid = 0;
  if (a.seg_desc) {
    // slot s holds rows (query token, head): row qi n_q + h of q_seq n_q
    const int seq = b / a.q_seq, qi = b - seq * a.q_seq;
    const int2 d = a.seg_desc[seq];
    const int slots = a.n_split + a.batch / a.q_seq;
    int s0 = 0;
    if (L > 0 && d.x >= 0 && d.x < slots) s0 = d.x, nvalid = min(d.y, min(slots - d.x, kMaxSplitsPerRow));
    nvalid = max(nvalid, 0);
    const int per_slot = a.q_seq * a.n_q;
    const int64_t first = (int64_t)s0 * per_slot + (int64_t)qi * a.n_q + h;
    o = reinterpret_cast<const uint4*>(wo + first * kRowBytes);
    m = a.ws_m + first;
    l = a.ws_l + first;
    ostep = per_slot * kUnits, mstep = per_slot, nload = nvalid;
  } else {
    o = reinterpret_cast<const uint4*>(wo + (int64_t)row * a.n_split * kRowBytes);
    m = a.ws_m + (int64_t)row * a.n_split;
    l = a.ws_l + (int64_t)row * a.n_split;
    ostep = kUnits, mstep = 1, nload = a.n_split;
  }
  uint4 v[kSteps][kCols];
  auto load_batch = [&](int s0) {
#pragma unroll
    for (int j = 0; j < kSteps; ++j) {
      const int s = s0 + j * kParts + part;
#pragma unroll
      for (int c = 0; c < kCols; ++c)
        v[j][c] = s < nload ? o[(int64_t)s * ostep + c * kLanesPerSplit + col] : uint4{0u, 0u, 0u, 0u};
    }
  };
  load_batch(0);
  float m0 = 0.f, l0 = 0.f;
  if (lane < nload) m0 = m[lane * mstep], l0 = l[lane * mstep];
  const float sink = a.sink ? a.sink[h] : kNegInf;

  if (!a.seg_desc) {
    const int per = ((L + a.n_split - 1) / a.n_split + 15) & ~15;  // split_chunk, in 32 bits
    nvalid = L == 0 ? 0 : (L + per - 1) / per;
  }

  // statistics: lane s holds split s (in chunks of 64)
  float M = sink;
  for (int c0 = 0; c0 < nvalid; c0 += 64) {
    const int s = c0 + lane;
    float mv = kNegInf, lv = 0.f;
    if (c0 == 0) {
      if (s < nvalid) mv = m0, lv = l0;
    } else if (s < nvalid) {
      mv = m[s * mstep], lv = l[s * mstep];
    }
    sm_m[wave][s] = mv;
    sm_w[wave][s] = lv;
    M = fmaxf(M, wave_max(mv));
  }
  float part_tot = 0.f;
  for (int c0 = 0; c0 < nvalid; c0 += 64) {
    const int s = c0 + lane;
    // a partial whose max is -inf (a masked query row) has weight 0, even when every one is
    const float w = s < nvalid && sm_m[wave][s] != kNegInf ? sm_w[wave][s] * fast_exp2((sm_m[wave][s] - M) * kLog2e) : 0.f;
    sm_w[wave][s] = w;
    part_tot += w;
  }
  float tot = wave_sum(part_tot);
  if (a.sink && M != kNegInf) tot += fast_exp2((sink - M) * kLog2e);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();

  typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
  // a unit's channels as floats
  auto unpack = [](const uint4& u, float (&f)[kE]) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
    if constexpr (H) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const f16x2_t x = __builtin_bit_cast(f16x2_t, w[k]);
        f[2 * k] = (float)x[0], f[2 * k + 1] = (float)x[1];
      }
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) f[k] = __uint_as_float(w[k]);
    }
  };
  float acc[kCols][kE];
#pragma unroll
  for (int c = 0; c < kCols; ++c)
#pragma unroll
    for (int e = 0; e < kE; ++e) acc[c][e] = 0.f;
  for (int s0 = 0; s0 < nvalid; s0 += kBatch) {
    if (s0 > 0) load_batch(s0);
#pragma unroll
    for (int j = 0; j < kSteps; ++j) {
      const int s = s0 + j * kParts + part;
      if (s < nvalid) {  // slots past nvalid hold stale or unwritten values
        const float w = sm_w[wave][s];
#pragma unroll
        for (int c = 0; c < kCols; ++c) {
          float f[kE];
          unpack(v[j][c], f);
#pragma unroll
          for (int e = 0; e < kE; ++e) acc[c][e] = fmaf(w, f[e], acc[c][e]);
        }
      }
    }
  }
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
#pragma unroll
  for (int c = 0; c < kCols; ++c) {
#pragma unroll
    for (int e = 0; e < kE; ++e) {
      float r = acc[c][e];
      if constexpr (kParts == 4) r = xor16_sum(r);
      if constexpr (kParts >= 2) r = xor32_sum(r);
      acc[c][e] = r * inv;
    }
    if (part == 0) {
#pragma unroll
      for (int k = 0; k < kE / 4; ++k)
        store4<OT>(a.out, (int64_t)row * VD + (c * kLanesPerSplit + col) * kE + 4 * k,
                   float4{acc[c][4 * k], acc[c][4 * k + 1], acc[c][4 * k + 2], acc[c][4 * k + 3]});
    }
  }
  if (a.lse && lane == 0) a.lse[row] = tot > 0.f ? M + __logf(tot) : kNegInf;
}

template <int DT>
__global__ void __launch_bounds__(256) update_kernel(const UpdateLaunch a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= a.rows) return;
  const int r = a.stat_stride;
  const float pm = a.prev_max[row * r], ps = a.prev_sum[row * r];
  const float cm = a.cur_max[row * r], cs = a.cur_sum[row * r];
  const float M = fmaxf(pm, cm);
  const float wp = pm == kNegInf ? 0.f : ps * fast_exp2((pm - M) * kLog2e);
  const float wc = cm == kNegInf ? 0.f : cs * fast_exp2((cm - M) * kLog2e);
  const float tot = wp + wc;
  const float fp = tot > 0.f ? wp / tot : 0.f;
  const float fc = tot > 0.f ? wc / tot : 0.f;
  const int64_t base = row * a.head_dim;
  for (int d = lane; d < a.head_dim; d += 64) {
    const float po = load_as_f32<DT>(a.prev_out, base + d);
    const float co = load_as_f32<DT>(a.cur_out, base + d);
    // an empty side contributes nothing, even if its buffer holds NaN
    float v = 0.f;
    if (fp != 0.f) v = fp * po;
    if (fc != 0.f) v = fmaf(fc, co, v);
    store_from_f32<DT>(a.out, base + d, v);
  }
  // all lanes have read their stats above; write after the row is done
  __builtin_amdgcn_wave_barrier();
  if (lane < r) {
    a.max_out[row * r + lane] = M;
    a.sum_out[row * r + lane] = tot;
  }
}

template <int VD, bool H>
hipError_t launch_combine_vd(const CombineLaunch& p, dim3 grid, hipStream_t stream) {
  switch (p.out_dtype) {
    case kF32: hipLaunchKernelGGL((combine_kernel<kF32, VD, H>), grid, dim3(256), 0, stream, p); break;
    case kF16: hipLaunchKernelGGL((combine_kernel<kF16, VD, H>), grid, dim3(256), 0, stream, p); break;
    case kBF16: hipLaunchKernelGGL((combine_kernel<kBF16, VD, H>), grid, dim3(256), 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Longest-first plan for one launch: one wave ranks all sequences.
__global__ void __launch_bounds__(64) plan_kernel(const int64_t* lens, int batch, int64_t cap, int2* plan) {
  __shared__ __attribute__((aligned(16))) uint32_t keys[kLongestFirstMaxBatch];
  int len[kLongestFirstMaxBatch / 64], rank[kLongestFirstMaxBatch / 64];
  rank_lengths(lens, batch, cap, keys, len, rank);
#pragma unroll
  for (int c = 0; c < kLongestFirstMaxBatch / 64; ++c)
    if (len[c] >= 0) plan[rank[c]] = int2{c * 64 + (int)threadIdx.x, len[c]};
}

}  // namespace

hipError_t launch_plan(const int64_t* seq_lens, int batch, int64_t cap, int2* plan, hipStream_t stream) {
  if (batch < 1 || batch > kLongestFirstMaxBatch) return hipErrorInvalidValue;
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(64), 0, stream, seq_lens, batch, cap, plan);
  return hipGetLastError();
}

hipError_t launch_combine(const CombineLaunch& p, hipStream_t stream) {
  const int64_t rows = (int64_t)p.batch * p.n_q;
  if (rows == 0) return hipSuccess;
  if (rows >= (int64_t)1 << 31) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock));
  if (p.n_split < 1 || p.n_split > kMaxSplitsPerRow) return hipErrorInvalidValue;
  if (p.o_f16) return p.v_dim == 512 ? launch_combine_vd<512, true>(p, grid, stream) : hipErrorInvalidValue;
  switch (p.v_dim) {
    case 64: return launch_combine_vd<64, false>(p, grid, stream);
    case 128: return launch_combine_vd<128, false>(p, grid, stream);
    case 512: return launch_combine_vd<512, false>(p, grid, stream);
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_update(const UpdateLaunch& p, hipStream_t stream) {
  if (p.rows == 0) return hipSuccess;
  const dim3 grid((unsigned)((p.rows + kRowsPerBlock - 1) / kRowsPerBlock));
  switch (p.dtype) {
    case kF32: hipLaunchKernelGGL(update_kernel<kF32>, grid, dim3(256), 0, stream, p); break;
    case kF16: hipLaunchKernelGGL(update_kernel<kF16>, grid, dim3(256), 0, stream, p); break;
    case kBF16: hipLaunchKernelGGL(update_kernel<kBF16>, grid, dim3(256), 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ifa
