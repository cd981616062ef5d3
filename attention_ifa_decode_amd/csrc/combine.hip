// Merge kernels (gfx950): the n-way combine of split partials with the
// learnable sink, and the pairwise RingAttentionUpdate.
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
// Both kernels are HBM-bound elementwise passes: one wave per row, lanes
// stride over the head dimension.
#include "common.hpp"
#include "kernels.hpp"

namespace ifa {
namespace {

constexpr int kRowsPerBlock = 4;

template <int OT>
__global__ void __launch_bounds__(256) combine_kernel(const CombineLaunch a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= (int64_t)a.batch * a.n_q) return;
  const int b = (int)(row / a.n_q), h = (int)(row % a.n_q);
  int64_t L = a.seq_lens[b];
  L = L < 0 ? 0 : (L > a.s_cap ? a.s_cap : L);
  const int64_t per = split_chunk(L, a.n_split);
  const int nvalid = L == 0 ? 0 : (int)((L + per - 1) / per);

  const float* m = a.ws_m + row * a.n_split;
  const float* l = a.ws_l + row * a.n_split;
  const float sink = a.sink ? a.sink[h] : kNegInf;
  float M = sink;
  for (int i = 0; i < nvalid; ++i) M = fmaxf(M, m[i]);
  float tot = (a.sink && M != kNegInf) ? fast_exp2((sink - M) * kLog2e) : 0.f;

  const float* o = a.ws_o + row * a.n_split * (int64_t)a.v_dim;
  const int64_t orow = row * a.v_dim;
  constexpr int kMaxPerLane = 8;  // v_dim <= 512
  float acc[kMaxPerLane];
#pragma unroll
  for (int k = 0; k < kMaxPerLane; ++k) acc[k] = 0.f;
  for (int i = 0; i < nvalid; ++i) {
    const float wgt = l[i] * fast_exp2((m[i] - M) * kLog2e);
    tot += wgt;
#pragma unroll
    for (int k = 0; k < kMaxPerLane; ++k) {
      const int d = lane + 64 * k;
      if (d < a.v_dim) acc[k] = fmaf(wgt, o[(int64_t)i * a.v_dim + d], acc[k]);
    }
  }
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
#pragma unroll
  for (int k = 0; k < kMaxPerLane; ++k) {
    const int d = lane + 64 * k;
    if (d < a.v_dim) store_from_f32<OT>(a.out, orow + d, acc[k] * inv);
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

}  // namespace

hipError_t launch_combine(const CombineLaunch& p, hipStream_t stream) {
  const int64_t rows = (int64_t)p.batch * p.n_q;
  if (rows == 0) return hipSuccess;
  if (p.v_dim > 512) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock));
  switch (p.out_dtype) {
    case kF32: hipLaunchKernelGGL(combine_kernel<kF32>, grid, dim3(256), 0, stream, p); break;
    case kF16: hipLaunchKernelGGL(combine_kernel<kF16>, grid, dim3(256), 0, stream, p); break;
    case kBF16: hipLaunchKernelGGL(combine_kernel<kBF16>, grid, dim3(256), 0, stream, p); break;
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
