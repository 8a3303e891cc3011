// Best-first draft-tree construction on gfx950: one wavefront per request (device code
// shared by the build kernel and the fused commit + next-build kernel).
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
// and the score of its next child (with the log-prob of the rank after it fetched ahead).  Each pop is a wave-wide fp64 max; ties go to the
// lowest lane, i.e. the smallest parent slot (and, within one parent, the smaller rank
// is the only one offered).  This pops exactly the sequence of a full frontier ordered by
// (score desc, parent asc, rank asc).  Only slots 0..63 can ever be parents (the 65th
// node is the last insertion), so 64 lanes suffice.

#pragma once

#include "gdntree_internal.h"

namespace gdntree {

struct BuildParams {
  const float *lat_logp;
  const int32_t *lat_tok, *root_tok;
  int P, K, N;
  gdntree_tree out;
  // draft positions per request [B], clipped to [0, P]; null: all P for every request
  const int32_t *positions = nullptr;
};

template <int CTRL, int ROWMASK>
__device__ __forceinline__ double dpp_max_f64(double x) {
  // y = x moved by the DPP pattern (lanes outside ROWMASK keep their own x), then max
  const long long bits = __double_as_longlong(x);
  const int lo = (int)(bits & 0xffffffffll), hi = (int)(bits >> 32);
  int ylo, yhi;
  if constexpr (ROWMASK == 0xf) {  // every lane is written: no old value needed
    ylo = __builtin_amdgcn_mov_dpp(lo, CTRL, 0xf, 0xf, true);
    yhi = __builtin_amdgcn_mov_dpp(hi, CTRL, 0xf, 0xf, true);
  } else {
    ylo = __builtin_amdgcn_update_dpp(lo, lo, CTRL, ROWMASK, 0xf, false);
    yhi = __builtin_amdgcn_update_dpp(hi, hi, CTRL, ROWMASK, 0xf, false);
  }
  const double y = __longlong_as_double(((long long)yhi << 32) | (long long)(unsigned)ylo);
  return y > x ? y : x;  // no NaN ever enters: candidates are finite or -inf
}

// fp32 maximum over the 64 lanes, returned uniformly: the same folding as the fp64 one, each
// step a single DPP max (inputs are finite or -inf, so no NaN handling is needed).  The
// s_nop before each step gives the two wait states a DPP read needs after a VALU write.
__device__ __forceinline__ float wave_max_f32(float x) {
  asm volatile(
      "s_nop 1\n\tv_max_f32_dpp %0, %0, %0 row_ror:1 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "s_nop 1\n\tv_max_f32_dpp %0, %0, %0 row_ror:2 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "s_nop 1\n\tv_max_f32_dpp %0, %0, %0 row_ror:4 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "s_nop 1\n\tv_max_f32_dpp %0, %0, %0 row_ror:8 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "s_nop 1\n\tv_max_f32_dpp %0, %0, %0 row_bcast:15 row_mask:0xa bank_mask:0xf\n\t"
      "s_nop 1\n\tv_max_f32_dpp %0, %0, %0 row_bcast:31 row_mask:0xc bank_mask:0xf\n\t"
      "s_nop 1"
      : "+v"(x));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}

__device__ __forceinline__ unsigned long long readlane_u64(unsigned long long x, int lane) {
  const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(x & 0xffffffffull), lane);
  const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(x >> 32), lane);
  return ((unsigned long long)hi << 32) | lo;
}

// Maximum over the 64 lanes, returned uniformly: row rotations (1, 2, 4, 8) give every lane
// its 16-lane row's maximum; two row broadcasts then fold rows 0..3 into lane 63.
__device__ __forceinline__ double wave_max_f64(double x) {
  x = dpp_max_f64<0x121, 0xf>(x);  // row_ror:1
  x = dpp_max_f64<0x122, 0xf>(x);  // row_ror:2
  x = dpp_max_f64<0x124, 0xf>(x);  // row_ror:4
  x = dpp_max_f64<0x128, 0xf>(x);  // row_ror:8
  x = dpp_max_f64<0x142, 0xa>(x);  // row_bcast:15 into rows 1, 3
  x = dpp_max_f64<0x143, 0xc>(x);  // row_bcast:31 into rows 2, 3
  const long long bits = __double_as_longlong(x);
  const int lo = __builtin_amdgcn_readlane((int)(bits & 0xffffffffll), 63);
  const int hi = __builtin_amdgcn_readlane((int)(bits >> 32), 63);
  return __longlong_as_double(((long long)hi << 32) | (long long)(unsigned)lo);
}

// Threads t = 0..nth-1 (of some part of the workgroup) copy request b's lattice into LDS:
// log-probs to s_logp and token ids to s_ltok (P * K entries each).
__device__ __forceinline__ void stage_lattice(const BuildParams &bp, int b, int t, int nth, float *s_logp,
                                              int *s_ltok) {
  const int PK = bp.P * bp.K;
  const float *lp = bp.lat_logp + (size_t)b * PK;
  const int32_t *lt = bp.lat_tok + (size_t)b * PK;
  for (int e = t; e < PK; e += nth) {
    s_logp[e] = lp[e];
    s_ltok[e] = lt[e];
  }
}

// Builds request b's tree.  Unless `staged` (the caller has staged the lattice with
// stage_lattice and met a workgroup barrier since), every thread of the workgroup (tid < nth)
// helps stage the lattice and meets the workgroup barrier; then the first wave alone runs the
// pops and writes the tree.
__device__ __forceinline__ void build_request(const BuildParams &bp, int b, int tid, int nth, float *s_logp,
                                              int *s_ltok, bool staged = false) {
  const int P = bp.P, K = bp.K, N = bp.N;
  // children are offered only at depths below this request's own position count
  const int Pb = bp.positions ? min(max(bp.positions[b], 0), P) : P;
  const gdntree_tree &out = bp.out;
  const int PK = P * K;
  if (!staged) {
    stage_lattice(bp, b, tid, nth, s_logp, s_ltok);
    __syncthreads();
  }
  if (tid >= 64) return;  // one wave builds
  const int lane = tid;
  const int root_token = bp.root_tok[b];  // loaded now, used after the pops
  // first-child log-prob of a node at depth d (children sit at lattice position d): lane d
  const float lp_first = s_logp[min(lane, P - 1) * K];

  // Lane l holds node l (its slot) and the one frontier candidate it offers (`has`): its
  // lowest unexpanded child rank `next`, that child's score `cand`, and, fetched ahead, the
  // log-prob `nlp` of the rank after it, so no LDS read sits between two pops.  Whether a
  // lane offers a candidate is a flag of its own: a candidate's score may be -inf (a log-prob
  // of -inf, or a finite fp64 sum that rounds to -inf in fp32) and is still a candidate.
  const double kNone = -__builtin_inf();
  int my_parent = -1, my_depth = 0, my_rank = -1, my_next = 0;
  double my_score = 0.0, cand = kNone;
  bool has = false;
  unsigned long long my_anc = 0ull;
  // LDS index of the fetched-ahead log-prob; every lane reloads its entry after each pop
  // (one unconditional read, so the value lands straight in its register)
  int nlp_at = 0;
  if (lane == 0) {  // the root (P >= 1 and K >= 1); no children when the request has no positions
    has = Pb > 0;
    cand = 0.0 + (double)s_logp[0];
    nlp_at = min(1, K - 1);
  }
  float nlp = s_logp[nlp_at];
  // The 65th slot (index 64) has no lane; it is the last insertion and is kept uniformly.
  int x_parent = -1, x_depth = 0, x_rank = -1;
  double x_score = 0.0;
  unsigned long long x_anc = 0ull;

  int n = 1;
  while (n <= N) {
    const double nlpd = (double)nlp;  // last use of the fetched-ahead value before it is refilled
    // The winner: rounding to fp32 is monotonic, so the fp64 maximum is among the offering
    // lanes whose rounded score equals the fp32 maximum; when that lane is unique it is the
    // winner, otherwise the exact fp64 maximum is taken over those lanes (ties to the lowest
    // lane, which holds the smallest parent slot).
    if (__ballot(has) == 0ull) break;                             // the trie is exhausted
    const float c32 = (float)cand;
    const float m32 = wave_max_f32(has ? c32 : -__builtin_inff());
    const bool top = has && c32 == m32;
    unsigned long long hit = __ballot(top);
    double m;
    if (__popcll(hit) == 1) {
      m = __longlong_as_double(readlane_u64((unsigned long long)__double_as_longlong(cand), __ffsll((long long)hit) - 1));
    } else {
      m = wave_max_f64(top ? cand : kNone);
      hit = __ballot(top && cand == m);
    }
    const int p = __ffsll((long long)hit) - 1;                    // smallest parent slot
    const int r = __builtin_amdgcn_readlane(my_next, p);
    const int dp = __builtin_amdgcn_readlane(my_depth, p);
    const int d = dp + 1;
    const unsigned long long a = readlane_u64(my_anc, p) | (1ull << (n - 1));
    const float first = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lp_first), min(d, P - 1)));

    // (fetched-ahead entries are clamped, always valid: one standing past the last rank or
    // position is never used)
    if (lane == p) {  // offer p's next child rank
      my_next = r + 1;
      has = r + 1 < K;
      cand = my_score + nlpd;
      nlp_at = dp * K + min(r + 2, K - 1);
    }
    if (n < 64) {
      if (lane == n) {
        my_parent = p; my_depth = d; my_rank = r; my_score = m; my_anc = a;
        my_next = 0;
        has = d < Pb;
        cand = m + (double)first;
        nlp_at = min(d, P - 1) * K + min(1, K - 1);
      }
    } else {
      x_parent = p; x_depth = d; x_rank = r; x_score = m; x_anc = a;
    }
    nlp = s_logp[nlp_at];
    ++n;
  }

  // tokens, after the build: the candidate of the node's rank at its lattice position
  const int *lt = s_ltok;
  const size_t base = (size_t)b * (N + 1);
  if (lane < n) {
    out.parent[base + lane] = my_parent;
    out.depth[base + lane] = my_depth;
    out.rank[base + lane] = my_rank;
    out.token[base + lane] = lane == 0 ? root_token : lt[(my_depth - 1) * K + my_rank];
    out.score[base + lane] = my_score;
    out.anc[base + lane] = my_anc;
  }
  if (lane == 0) {
    if (n == 65) {
      out.parent[base + 64] = x_parent;
      out.depth[base + 64] = x_depth;
      out.rank[base + 64] = x_rank;
      out.token[base + 64] = lt[(x_depth - 1) * K + x_rank];
      out.score[base + 64] = x_score;
      out.anc[base + 64] = x_anc;
    }
    out.n_nodes[b] = n;
  }
}

}  // namespace gdntree
