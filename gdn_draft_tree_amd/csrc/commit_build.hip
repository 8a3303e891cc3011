// One launch that commits a step's accepted-path states and builds the next step's draft tree.
//
// The two are independent: the commit is bound by the state's HBM traffic and uses every CU,
// the build is a latency-bound chain of one wave per request that moves almost no data.
// Run back to back, the build's ~20 us leave the memory system idle; in one launch the
// build's workgroups come first in the grid, so they are dispatched first and their waves
// run (at raised issue priority) beside the commit's.  The caller orders the launch after
// the step's acceptance, which is what the next draft (and so the next build) needs.

#include "build_device.h"
#include "commit_device.h"

namespace gdntree {
namespace {

template <int D, bool BF16IN>
__global__ __launch_bounds__(256) void commit_build_kernel(CommitParams p, BuildParams bp, int nb) {
  __shared__ CommitSmem<D> sm;
  __shared__ float s_logp[kMaxP * kMaxK];
  if ((int)blockIdx.x < nb) {
    __builtin_amdgcn_s_setprio(2);
    build_request(bp, blockIdx.x, threadIdx.x, 256, s_logp);
    return;
  }
  commit_unit<D, BF16IN, false>(p, blockIdx.x - nb, threadIdx.x, sm);
}

template <int D, bool BF16IN>
hipError_t launch_cb(const CommitParams &p, const BuildParams &bp, int nb, hipStream_t stream) {
  const long long blocks = (long long)nb + (long long)p.L * p.B * p.H * (D / 32);
  hipLaunchKernelGGL((commit_build_kernel<D, BF16IN>), dim3((unsigned)blocks), dim3(256), 0, stream, p, bp, nb);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_commit_build(const CommitParams &p, const BuildParams &bp, int nb, hipStream_t stream) {
  if (p.D == 64) return p.in_bf16 ? launch_cb<64, true>(p, bp, nb, stream) : launch_cb<64, false>(p, bp, nb, stream);
  return p.in_bf16 ? launch_cb<128, true>(p, bp, nb, stream) : launch_cb<128, false>(p, bp, nb, stream);
}

}  // namespace gdntree
