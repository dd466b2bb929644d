// debug_checks.hip -- device-side input checks used by the debug build of the
// library (libcsa_debug.so, csa_api.hip compiled with CSA_DEBUG).
//
// An attention index row holds pool-entry ids in [0, T) and -1 for an empty
// slot (page "DeepSeek-V4", section "Attention mask layout": slots that cannot
// be filled carry the -1 sentinel).  The kernels already treat any other value
// as an empty slot; the debug build reports it instead.
#include <climits>

#include "csa_device.hpp"

namespace csa {
namespace {

// res[0]: number of entries outside [-1, T); res[1]: the smallest such element
// index (both set by the caller to 0 and INT_MAX first)
__global__ __launch_bounds__(256) void check_idx_kernel(const int* __restrict__ idx, long n,
                                                        int T, int* __restrict__ res) {
  for (long i = blockIdx.x * 256L + threadIdx.x; i < n; i += (long)gridDim.x * 256L) {
    const int v = idx[i];
    if (v < -1 || v >= T) {
      atomicAdd(&res[0], 1);
      atomicMin(&res[1], (int)(i < (long)INT_MAX ? i : (long)INT_MAX));
    }
  }
}

}  // namespace

hipError_t launch_check_idx(const int* idx, long n, int T, int* res, hipStream_t s) {
  long blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(check_idx_kernel, dim3((unsigned)blocks), dim3(256), 0, s, idx, n, T, res);
  return hipGetLastError();
}

}  // namespace csa
