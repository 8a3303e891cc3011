// Best-first draft-tree construction on gfx950: one wavefront per request.
//
// Follows the SpecPilot summary (Prerequisites > draft-tree verification: nodes are added
// greedily by path log-prob until N; Technical novelty: edges scored by log p(child |
// parent)).  A node's score is its parent's score plus the fp32 lattice log-prob of its
// rank at its position, added in fp64, so every score is bit-identical to a root-to-leaf
// fp64 summation.
//
// Frontier.  Because each position's candidates are sorted by non-increasing log-prob,
// the best not-yet-inserted child of an inserted node p is always its lowest-rank one.
// So the frontier needs one candidate per inserted node: lane p of the wave holds node p
// and the score of its next child.  Each pop is a wave-wide fp64 max; ties go to the
// lowest lane, i.e. the smallest parent slot (and, within one parent, the smaller rank
// is the only one offered).  This pops exactly the sequence of a full frontier ordered by
// (score desc, parent asc, rank asc).  Only slots 0..63 can ever be parents (the 65th
// node is the last insertion), so 64 lanes suffice.

#include "gdntree_internal.h"

namespace gdntree {
namespace {

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x) {
  const long long bits = __double_as_longlong(x);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(bits & 0xffffffffll), CTRL, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(bits >> 32), CTRL, 0xf, 0xf, false);
  return __longlong_as_double(((long long)hi << 32) | (long long)(unsigned)lo);
}

__device__ __forceinline__ double readlane_f64(double x, int lane) {
  const long long bits = __double_as_longlong(x);
  const int lo = __builtin_amdgcn_readlane((int)(bits & 0xffffffffll), lane);
  const int hi = __builtin_amdgcn_readlane((int)(bits >> 32), lane);
  return __longlong_as_double(((long long)hi << 32) | (long long)(unsigned)lo);
}

__device__ __forceinline__ unsigned long long readlane_u64(unsigned long long x, int lane) {
  const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(x & 0xffffffffull), lane);
  const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(x >> 32), lane);
  return ((unsigned long long)hi << 32) | lo;
}

// Maximum over the 64 lanes.  Row rotations (DPP row_ror 1, 2, 4, 8) leave every lane
// holding its 16-lane row's maximum; the four row maxima are then combined uniformly.
__device__ __forceinline__ double wave_max_f64(double x) {
  x = fmax(x, dpp_f64<0x121>(x));
  x = fmax(x, dpp_f64<0x122>(x));
  x = fmax(x, dpp_f64<0x124>(x));
  x = fmax(x, dpp_f64<0x128>(x));
  const double r0 = readlane_f64(x, 0), r1 = readlane_f64(x, 16);
  const double r2 = readlane_f64(x, 32), r3 = readlane_f64(x, 48);
  return fmax(fmax(r0, r1), fmax(r2, r3));
}

__global__ __launch_bounds__(64) void build_tree_kernel(const float *__restrict__ lat_logp,
                                                         const int32_t *__restrict__ lat_tok,
                                                         const int32_t *__restrict__ root_tok,
                                                         int P, int K, int N, gdntree_tree out) {
  __shared__ float s_logp[kMaxP * kMaxK];
  __shared__ int32_t s_tok[kMaxP * kMaxK];

  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const int PK = P * K;
  const float *lp = lat_logp + (size_t)b * PK;
  const int32_t *lt = lat_tok + (size_t)b * PK;
  for (int e = lane; e < PK; e += 64) {
    s_logp[e] = lp[e];
    s_tok[e] = lt[e];
  }
  __syncthreads();

  // Node held by this lane (slot == lane) and the score of its next child candidate.
  int my_parent = -1, my_depth = 0, my_rank = -1, my_token = 0, my_next = 0;
  double my_score = 0.0, my_cand = 0.0;
  unsigned long long my_anc = 0ull;
  bool has_cand = false;
  if (lane == 0) {
    my_token = root_tok[b];
    has_cand = true;  // P >= 1 and K >= 1
    my_cand = 0.0 + (double)s_logp[0];
  }
  // The 65th slot (index 64) has no lane; its fields are kept uniformly.
  int x_parent = -1, x_depth = 0, x_rank = -1, x_token = 0;
  double x_score = 0.0;
  unsigned long long x_anc = 0ull;

  int n = 1;
  while (n <= N) {
    const unsigned long long valid = __ballot(has_cand);
    if (valid == 0ull) break;
    const double c = has_cand ? my_cand : -__builtin_inf();
    const double m = wave_max_f64(c);
    const unsigned long long hit = __ballot(has_cand && c == m);
    const int p = __ffsll((long long)hit) - 1;                  // smallest parent slot
    const double sc = readlane_f64(c, p);                        // bit-exact winning score
    const int r = __builtin_amdgcn_readlane(my_next, p);
    const int d = __builtin_amdgcn_readlane(my_depth, p) + 1;
    const unsigned long long a = readlane_u64(my_anc, p) | (1ull << (n - 1));
    const int tok = s_tok[(d - 1) * K + r];

    if (lane == p) {  // offer p's next sibling of the popped child
      my_next = r + 1;
      has_cand = my_next < K;
      if (has_cand) my_cand = my_score + (double)s_logp[my_depth * K + my_next];
    }
    if (n < 64) {
      if (lane == n) {
        my_parent = p; my_depth = d; my_rank = r; my_token = tok; my_score = sc; my_anc = a;
        my_next = 0;
        has_cand = d < P;
        if (has_cand) my_cand = sc + (double)s_logp[d * K];
      }
    } else {
      x_parent = p; x_depth = d; x_rank = r; x_token = tok; x_score = sc; x_anc = a;
    }
    ++n;
  }

  const size_t base = (size_t)b * (N + 1);
  if (lane < n) {
    out.parent[base + lane] = my_parent;
    out.depth[base + lane] = my_depth;
    out.rank[base + lane] = my_rank;
    out.token[base + lane] = my_token;
    out.score[base + lane] = my_score;
    out.anc[base + lane] = my_anc;
  }
  if (lane == 0) {
    if (n == 65) {
      out.parent[base + 64] = x_parent;
      out.depth[base + 64] = x_depth;
      out.rank[base + 64] = x_rank;
      out.token[base + 64] = x_token;
      out.score[base + 64] = x_score;
      out.anc[base + 64] = x_anc;
    }
    out.n_nodes[b] = n;
  }
}

}  // namespace

hipError_t launch_build(const float *lat_logp, const int32_t *lat_tok, const int32_t *root_tok,
                        int B, int P, int K, int N, gdntree_tree out, hipStream_t stream) {
  hipLaunchKernelGGL(build_tree_kernel, dim3(B), dim3(64), 0, stream, lat_logp, lat_tok,
                     root_tok, P, K, N, out);
  return hipGetLastError();
}

}  // namespace gdntree
