// One launch that commits a step's accepted-path states and builds the next step's draft tree
// (optionally with the step's acceptance in the same launch).
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
__global__ __launch_bounds__(256, kCommitWavesPerEU) void commit_build_kernel(CommitParams p, BuildParams bp, int nb) {
  __shared__ CommitSmem<D> sm;
  __shared__ float s_logp[kMaxP * kMaxK];
  __shared__ int s_ltok[kMaxP * kMaxK];
  if ((int)blockIdx.x < nb) {
    __builtin_amdgcn_s_setprio(2);
    build_request(bp, blockIdx.x, threadIdx.x, 256, s_logp, s_ltok);
    return;
  }
  commit_unit<D, BF16IN, kPathGiven>(p, blockIdx.x - nb, threadIdx.x, sm);
}

// Acceptance, commit and the next build in one launch.  Workgroup b < max(B, nb) first walks
// request b's acceptance (b < B) and writes it, then builds request b's next tree (b < nb):
// each request's next build starts once its own acceptance is known.  The commit workgroups
// walk their request's tree themselves.
template <int D, bool BF16IN>
__global__ __launch_bounds__(256, kCommitWavesPerEU) void accept_commit_build_kernel(CommitParams p, BuildParams bp, int nb, int na) {
  __shared__ CommitSmem<D> sm;
  __shared__ float s_logp[kMaxP * kMaxK];
  __shared__ int s_ltok[kMaxP * kMaxK];
  const int b = blockIdx.x, tid = threadIdx.x;
  if (b < na) {
    __builtin_amdgcn_s_setprio(2);
    // waves 1-3 fetch the next lattice (an input of this launch) while wave 0 walks, so the
    // build after the walk starts with its log-probs already in LDS
    if (b < nb && tid >= 64) stage_lattice(bp, b, tid - 64, 192, s_logp, s_ltok);
    if (b < p.B && tid < 64) accept_walk(p, b, tid, sm.path, sm.tok, &sm.len, &sm.bonus);
    __syncthreads();
    if (b < p.B && tid <= p.P && sm.len != 0) write_acceptance(p, b, tid, sm.len, sm.path, sm.tok, sm.bonus);
    if (b < nb) build_request(bp, b, tid, 256, s_logp, s_ltok, true);
    return;
  }
  commit_unit<D, BF16IN, kWalk>(p, b - na, tid, sm);
}

template <int D, bool BF16IN>
hipError_t launch_acb(const CommitParams &p, const BuildParams &bp, int nb, hipStream_t stream) {
  const int na = nb > p.B ? nb : p.B;
  const long long blocks = (long long)na + (long long)p.L * p.B * p.H;
  hipLaunchKernelGGL((accept_commit_build_kernel<D, BF16IN>), dim3((unsigned)blocks), dim3(256), 0, stream, p, bp,
                     nb, na);
  return hipGetLastError();
}

template <int D, bool BF16IN>
hipError_t launch_cb(const CommitParams &p, const BuildParams &bp, int nb, hipStream_t stream) {
  const long long blocks = (long long)nb + (long long)p.L * p.B * p.H;
  hipLaunchKernelGGL((commit_build_kernel<D, BF16IN>), dim3((unsigned)blocks), dim3(256), 0, stream, p, bp, nb);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_accept_commit_build(const CommitParams &p, const BuildParams &bp, int nb, hipStream_t stream) {
  if (p.D == 64) return p.in_bf16 ? launch_acb<64, true>(p, bp, nb, stream) : launch_acb<64, false>(p, bp, nb, stream);
  return p.in_bf16 ? launch_acb<128, true>(p, bp, nb, stream) : launch_acb<128, false>(p, bp, nb, stream);
}

hipError_t launch_commit_build(const CommitParams &p, const BuildParams &bp, int nb, hipStream_t stream) {
  if (p.D == 64) return p.in_bf16 ? launch_cb<64, true>(p, bp, nb, stream) : launch_cb<64, false>(p, bp, nb, stream);
  return p.in_bf16 ? launch_cb<128, true>(p, bp, nb, stream) : launch_cb<128, false>(p, bp, nb, stream);
}

}  // namespace gdntree
