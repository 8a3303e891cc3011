// Best-first draft trees for a whole batch under one shared node budget, on gfx950.
//
// SpecPilot summary, Technical novelty (batching: the budget of draft rows is shared by the
// batch, and each request gets its own number of draft positions).  One best-first pass
// over the union of the requests' frontiers adds the batch's best candidate until the batch
// holds G draft nodes; a request holding N drafts offers no more; ties go to the smaller
// request, then the smaller parent slot, then the smaller rank.
//
// Why two short launches reach exactly that: a request's candidates never depend on another
// request's pops, and its own best-first sequence has non-increasing scores (log-probs are
// <= 0, so a child never outscores its parent).  So the batch pass pops, at every step, the
// best head among the requests' own sequences, i.e. it takes the first G elements of their
// merge under (score desc, request asc, slot asc), and every request keeps a prefix of its
// own tree.  The per-request trees are built first, one wave each and capped at N
// (build_device.h); then one workgroup merges the requests' score lists pairwise in a tree of
// merges, keeping only the first G keys of every merged list (the batch's first G lie among
// the first G of any part), and counts each request's keys among the first G of the last
// list.  Each merged key is placed by its own thread with a binary search along the merge
// path, so a level of the tree is one pass and one barrier.  Slots at or past the new node
// count keep what the build wrote there; like every unused slot they are never read.

#include "build_device.h"

namespace gdntree {
namespace {

constexpr int kSelThreads = 1024;

// Bp: B rounded up to a power of two; 1 <= G < B * N; Bp * min(N, G) <= kSharedMaxSlots.
// Keys are the scores: every merge joins a list A of lower requests with a list C of higher
// ones, so on equal scores A's key comes first, and within one list equal scores keep slot
// order; each key carries its request (-1 for a sentinel, a slot that holds no node), and a
// sentinel comes after every real key, one scored -inf included.
__device__ __forceinline__ bool key_first(double ka, int ra, double kc, int rc) {
  if (rc < 0) return true;   // C is a sentinel: A (real or not) comes first
  if (ra < 0) return false;  // A is a sentinel, C is real
  return ka >= kc;
}
__global__ __launch_bounds__(kSelThreads) void select_budget_kernel(const double *score, int32_t *n_nodes,
                                                                    int B, int Bp, int N, int G) {
  __shared__ double s_key[2][kSharedMaxSlots];
  __shared__ short s_req[2][kSharedMaxSlots];
  __shared__ int s_cnt[kSharedMaxB];
  const int tid = threadIdx.x;
  // level 0: Bp lists (the requests, then empty ones) of their first len0 draft slots.  Every
  // load is issued before any is used (a slot's score is read whether or not it holds a node:
  // it lies inside the [B][N+1] tree either way), so level 0 waits for one memory latency.
  const int len0 = N < G ? N : G;
  constexpr int kPer = kSharedMaxSlots / kSelThreads;
  double sv[kPer];
  int room[kPer];
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int e = tid + r * kSelThreads, j = e / len0, i = e % len0;
    sv[r] = -__builtin_inf();
    room[r] = 0;
    if (e < Bp * len0 && j < B) {
      sv[r] = score[(size_t)j * (N + 1) + i + 1];
      room[r] = n_nodes[j] - 1 - i;  // > 0 iff slot i + 1 holds a node
    }
  }
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int e = tid + r * kSelThreads;
    if (e < Bp * len0) {
      const bool real = room[r] > 0;
      s_key[0][e] = real ? sv[r] : -__builtin_inf();
      s_req[0][e] = (short)(real ? e / len0 : -1);
    }
  }
  for (int b = tid; b < B; b += kSelThreads) s_cnt[b] = 0;
  __syncthreads();

  int cur = 0, nl = Bp, len = len0;
  while (nl > 1) {
    const int nlen = 2 * len < G ? 2 * len : G;
    const double *ks = s_key[cur];
    const short *rq = s_req[cur];
    for (int t = tid; t < (nl / 2) * nlen; t += kSelThreads) {
      const int m = t / nlen, k = t % nlen;
      const int a0 = 2 * m * len, c0 = a0 + len;  // lists A = [a0, a0 + len) and C = [c0, c0 + len)
      // i = how many of the first k merged keys come from A: the first i whose A[i] does not
      // come before C[k - 1 - i]
      int lo = k > len ? k - len : 0, hi = k < len ? k : len;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (key_first(ks[a0 + mid], rq[a0 + mid], ks[c0 + k - 1 - mid], rq[c0 + k - 1 - mid])) lo = mid + 1;
        else hi = mid;
      }
      const int i = lo, j = k - lo;
      const int src = (i < len && (j >= len || key_first(ks[a0 + i], rq[a0 + i], ks[c0 + j], rq[c0 + j]))) ? a0 + i : c0 + j;
      s_key[cur ^ 1][t] = ks[src];
      s_req[cur ^ 1][t] = s_req[cur][src];
    }
    __syncthreads();
    cur ^= 1;
    nl >>= 1;
    len = nlen;
  }

  // every real key among the first G joins its request's count
  const int take = G < len ? G : len;
  for (int e = tid; e < take; e += kSelThreads)
    if (s_req[cur][e] >= 0) atomicAdd(&s_cnt[s_req[cur][e]], 1);
  __syncthreads();
  for (int b = tid; b < B; b += kSelThreads) n_nodes[b] = 1 + s_cnt[b];
}

// G == 0: every request keeps its root alone
__global__ __launch_bounds__(256) void roots_only_kernel(int32_t *n_nodes, int B) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b < B) n_nodes[b] = 1;
}

}  // namespace

int shared_budget_lists(int B) {
  int Bp = 1;
  while (Bp < B) Bp <<= 1;
  return Bp;
}

hipError_t launch_budget_cut(const gdntree_tree &out, int B, int N, int G, hipStream_t stream) {
  if (G >= B * N) return hipSuccess;  // no request is cut: the independent builds are the answer
  if (G == 0) {
    hipLaunchKernelGGL(roots_only_kernel, dim3((B + 255) / 256), dim3(256), 0, stream, out.n_nodes, B);
  } else {
    hipLaunchKernelGGL(select_budget_kernel, dim3(1), dim3(kSelThreads), 0, stream, (const double *)out.score,
                       out.n_nodes, B, shared_budget_lists(B), N, G);
  }
  return hipGetLastError();
}

hipError_t launch_build_shared(const BuildParams &bp, int B, int G, hipStream_t stream) {
  hipError_t e = launch_build_params(bp, B, stream);
  if (e != hipSuccess) return e;
  return launch_budget_cut(bp.out, B, bp.N, G, stream);
}

}  // namespace gdntree
