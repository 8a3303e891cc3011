// Best-first draft-tree construction on gfx950: one wavefront per request (the pops are
// in build_device.h).

#include "build_device.h"

namespace gdntree {
namespace {

__global__ __launch_bounds__(64) void build_tree_kernel(BuildParams bp) {
  __shared__ float s_logp[kMaxP * kMaxK];
  __shared__ int s_ltok[kMaxP * kMaxK];
  build_request(bp, blockIdx.x, threadIdx.x, 64, s_logp, s_ltok);
}

}  // namespace

hipError_t launch_build_params(const BuildParams &bp, int B, hipStream_t stream) {
  hipLaunchKernelGGL(build_tree_kernel, dim3(B), dim3(64), 0, stream, bp);
  return hipGetLastError();
}

hipError_t launch_build(const float *lat_logp, const int32_t *lat_tok, const int32_t *root_tok,
                        int B, int P, int K, int N, gdntree_tree out, hipStream_t stream) {
  const BuildParams bp{lat_logp, lat_tok, root_tok, P, K, N, out, nullptr};
  return launch_build_params(bp, B, stream);
}

}  // namespace gdntree
