// MLA-shaped split-KV decode (MFMA path): not built yet.
#include "common.hpp"
#include "kernels.hpp"

namespace ifa {

hipError_t launch_mla_splitkv(const MlaLaunch& p, hipStream_t stream) {
  (void)p;
  (void)stream;
  return hipErrorNotSupported;
}

}  // namespace ifa
