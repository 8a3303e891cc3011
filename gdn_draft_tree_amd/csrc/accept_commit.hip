// Acceptance, and the accepted-path commit (device code in commit_device.h).

#include "commit_device.h"

namespace gdntree {
namespace {

__global__ __launch_bounds__(64) void accept_kernel(CommitParams p) {
  __shared__ int s_path[kMaxAnc];
  __shared__ int s_tok[kMaxSlots];
  __shared__ int s_len, s_bonus;
  const int b = blockIdx.x, lane = threadIdx.x;
  accept_walk(p, b, lane, s_path, s_tok, &s_len, &s_bonus);
  __syncthreads();
  const int len = s_len;
  if (len == 0) return;  // malformed node count: nothing is written
  if (lane <= p.P) write_acceptance(p, b, lane, len, s_path, s_tok, s_bonus);
}

template <int D, bool BF16IN, int PATH>
__global__ __launch_bounds__(256, kCommitWavesPerEU) void commit_kernel(CommitParams p) {
  __shared__ CommitSmem<D> sm;
  commit_unit<D, BF16IN, PATH>(p, blockIdx.x, threadIdx.x, sm);
}

template <int D, bool BF16IN, int PATH>
hipError_t launch_d(const CommitParams &p, hipStream_t stream) {
  const long long blocks = (long long)p.L * p.B * p.H;
  hipLaunchKernelGGL((commit_kernel<D, BF16IN, PATH>), dim3((unsigned)blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <int PATH>
hipError_t launch_w(const CommitParams &p, hipStream_t stream) {
  if (p.D == 64) return p.in_bf16 ? launch_d<64, true, PATH>(p, stream) : launch_d<64, false, PATH>(p, stream);
  return p.in_bf16 ? launch_d<128, true, PATH>(p, stream) : launch_d<128, false, PATH>(p, stream);
}

}  // namespace

hipError_t launch_accept_commit(const CommitParams &p, hipStream_t stream) { return launch_w<kWalkAndWrite>(p, stream); }

hipError_t launch_commit(const CommitParams &p, hipStream_t stream) { return launch_w<kPathGiven>(p, stream); }

hipError_t launch_accept(const CommitParams &p, hipStream_t stream) {
  hipLaunchKernelGGL(accept_kernel, dim3((unsigned)p.B), dim3(64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace gdntree
