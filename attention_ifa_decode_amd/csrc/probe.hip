// Read-stream probe (gfx950): the HBM read rate one launch sustains on this
// GPU, measured beside the decode so that its achieved bandwidth can be set
// against a ceiling taken on the same device in the same run.
//
// Every 16-byte chunk of the buffer is read exactly once with non-temporal
// vector loads, 8 per lane in flight; lane i of the grid takes chunks
// i, i + G, i + 2G, ... (G = grid lanes), so each wave-wide load covers 1 KB
// of consecutive bytes.  The XOR of the words read is stored per workgroup,
// which keeps every load live and writes only 4 bytes per workgroup.
#include "common.hpp"
#include "kernels.hpp"

namespace ifa {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kInFlight = 8;

__global__ void __launch_bounds__(kProbeThreads) read_stream_kernel(const u32x4* p, uint64_t n, uint32_t* out) {
  const uint64_t stride = (uint64_t)gridDim.x * kProbeThreads;
  uint64_t i = (uint64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kInFlight - 1) * stride < n; i += kInFlight * stride) {
    u32x4 v[kInFlight];
#pragma unroll
    for (int k = 0; k < kInFlight; ++k) v[k] = __builtin_nontemporal_load(p + i + k * stride);
#pragma unroll
    for (int k = 0; k < kInFlight; ++k) acc ^= word(v[k], 0) ^ word(v[k], 1) ^ word(v[k], 2) ^ word(v[k], 3);
  }
  for (; i < n; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(p + i);
    acc ^= word(v, 0) ^ word(v, 1) ^ word(v, 2) ^ word(v, 3);
  }
  // one value per workgroup: the XOR over its lanes
  __shared__ uint32_t sm[kProbeThreads];
  sm[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t x = 0;
    for (int k = 0; k < kProbeThreads; ++k) x ^= sm[k];
    out[blockIdx.x] = x;
  }
}

}  // namespace

hipError_t launch_read_probe(const void* buf, uint64_t bytes, uint32_t* out, int workgroups, hipStream_t stream) {
  hipLaunchKernelGGL(read_stream_kernel, dim3(workgroups), dim3(kProbeThreads), 0, stream,
                     static_cast<const u32x4*>(buf), bytes / 16, out);
  return hipGetLastError();
}

}  // namespace ifa
