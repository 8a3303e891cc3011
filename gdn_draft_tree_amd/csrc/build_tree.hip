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

// Parent-conditioned rows: four waves stage and sort the request's P * K rows, then the first
// wave builds.
__global__ __launch_bounds__(256) void build_cond_kernel(BuildParams bp) {
  // the sorted rows, then the unsorted ones (P * K * K entries each, at the request's P and K)
  __shared__ alignas(16) float s_rows[2 * kMaxP * kCondMaxK * kCondMaxK];
  __shared__ uint8_t s_perm[kMaxP * kCondMaxK * kCondMaxK];
  __shared__ int s_ltok[kMaxP * kCondMaxK];
  float *s_logp = s_rows, *s_raw = s_rows + bp.P * bp.K * bp.K;
  stage_lattice_cond(bp, blockIdx.x, threadIdx.x, 256, s_raw, s_logp, s_perm, s_ltok);
  build_request<true>(bp, blockIdx.x, threadIdx.x, 256, s_logp, s_ltok, true, s_perm);
}

}  // namespace

hipError_t launch_build_params(const BuildParams &bp, int B, hipStream_t stream) {
  hipLaunchKernelGGL(build_tree_kernel, dim3(B), dim3(64), 0, stream, bp);
  return hipGetLastError();
}

hipError_t launch_build_cond(const float *edge_logp, const int32_t *lat_tok, const int32_t *root_tok, int B,
                             int P, int K, int N, gdntree_tree out, hipStream_t stream) {
  BuildParams bp{nullptr, lat_tok, root_tok, P, K, N, out, nullptr};
  bp.edge_logp = edge_logp;
  hipLaunchKernelGGL(build_cond_kernel, dim3(B), dim3(256), 0, stream, bp);
  return hipGetLastError();
}

hipError_t launch_build(const float *lat_logp, const int32_t *lat_tok, const int32_t *root_tok,
                        int B, int P, int K, int N, gdntree_tree out, hipStream_t stream) {
  const BuildParams bp{lat_logp, lat_tok, root_tok, P, K, N, out, nullptr};
  return launch_build_params(bp, B, stream);
}

}  // namespace gdntree
