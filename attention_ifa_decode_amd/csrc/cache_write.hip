// Paged KV-cache write (gfx950): the step just before a decode step, which
// places each new token's K/V rows into the block pool.
//
// aclnnMlaPrologV3WeightNz, "Parameters": kvCacheRef and krCacheRef are
// updated in place at the slots cacheIndexOptional names (CacheMode PA_BSND:
// slot s in [0, BlockNum * BlockSize) is position s % BlockSize of block
// s / BlockSize).  A plain copy: every 16-byte chunk of a source row is one
// lane's load and store, consecutive lanes take consecutive chunks, so both
// sides are coalesced.  HBM-bound: T * N_kv * D * esz bytes read and written.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.hpp"

namespace ifa {
namespace {

__global__ void __launch_bounds__(256) cache_write_kernel(const CacheWriteLaunch p) {
  const int64_t chunks = p.row_chunks;  // 16-byte chunks per (token, head) row
  const int64_t total = p.tokens * p.n_kv * chunks;
  const int64_t pool_slots = p.num_blocks * p.block_size;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int64_t c = i % chunks;
    const int64_t tg = i / chunks;
    const int64_t g = tg % p.n_kv, t = tg / p.n_kv;
    const int64_t slot = p.slot_index[t];
    if (slot < 0 || slot >= pool_slots) continue;  // outside the pool: skipped
    const int64_t row = p.token_major ? slot * p.n_kv + g
                                      : ((slot / p.block_size) * p.n_kv + g) * p.block_size + slot % p.block_size;
    const uint4 v = reinterpret_cast<const uint4*>(p.src)[i];
    *reinterpret_cast<uint4*>(static_cast<char*>(p.cache) + row * p.row_bytes + p.col_bytes + c * 16) = v;
  }
}

}  // namespace

hipError_t launch_cache_write(const CacheWriteLaunch& p, hipStream_t stream) {
  const int64_t total = p.tokens * p.n_kv * p.row_chunks;
  if (total == 0) return hipSuccess;
  int64_t grid = (total + 255) / 256;
  if (grid > 4096) grid = 4096;
  hipLaunchKernelGGL(cache_write_kernel, dim3((unsigned)grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace ifa
