// Input check of a decode call: the lengths and the block-table entries it
// would read.  The decode itself clamps a length to [0, capacity] and a block
// id to [0, num_blocks), so that a corrupt argument never leads it outside its
// buffers; this kernel reports such arguments instead of hiding them.
//
// One workgroup: thread i takes sequences i, i + 1024, ...; for each, the
// length and the entries block_table[b][0 .. ceil(clamped length / block
// size) - 1].  The flags of all threads are OR-ed through LDS and thread 0
// writes the one result word (no atomics, nothing to zero beforehand).
#include "common.hpp"
#include "kernels.hpp"

namespace ifa {
namespace {

constexpr int kCheckThreads = 1024;

__global__ void __launch_bounds__(kCheckThreads) check_inputs_kernel(const CheckLaunch a) {
  __shared__ uint32_t sm[kCheckThreads];
  uint32_t f = 0;
  for (int64_t b = threadIdx.x; b < a.batch; b += kCheckThreads) {
    const int64_t L = a.seq_lens[b];
    if (L < 0 || L > a.s_cap) f |= kCheckBadLength;
    if (a.block_table != nullptr) {
      const int64_t Lc = L < 0 ? 0 : (L > a.s_cap ? a.s_cap : L);
      const int64_t nb = (Lc + a.block_size - 1) / a.block_size;  // <= max_blocks, as s_cap = max_blocks * block_size
      const int32_t* row = a.block_table + b * a.max_blocks;
      for (int64_t j = 0; j < nb; ++j) {
        const int32_t v = row[j];
        if (v < 0 || v >= a.num_blocks) f |= kCheckBadBlock;
      }
    }
  }
  sm[threadIdx.x] = f;
  __syncthreads();
  for (int s = kCheckThreads / 2; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) sm[threadIdx.x] |= sm[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) *a.flags = (int32_t)sm[0];
}

}  // namespace

hipError_t launch_check(const CheckLaunch& p, hipStream_t stream) {
  hipLaunchKernelGGL(check_inputs_kernel, dim3(1), dim3(kCheckThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace ifa
