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
//
// Parent-conditioned edges (a Markov-head lattice: the log-prob of child rank r at position s
// depends on the parent's own rank pr at position s-1).  Each (s, pr) row of log-probs is
// sorted once (descending, equal values by rank) with the permutation kept, and a node
// offers its children in its own row's order: the same frontier argument holds row by row,
// and the plain lattice is the special case of one row per position.  Row order is the
// (sum desc, rank asc) order of the children as long as distinct log-probs give distinct
// fp64 sums with the node's score; a node scored -inf, whose children all tie at -inf,
// offers them in rank order instead (from the unsorted row).

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
  // parent-conditioned edge log-probs [B][P][K][K] ([b][s][pr][r]); null: the plain lattice
  const float *edge_logp = nullptr;
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

// Threads t = 0..nth-1 stage request b's parent-conditioned rows: the raw rows to s_raw, then
// (after a workgroup barrier) every row sorted by descending log-prob, equal values by rank,
// to s_logp with the permutation (the candidate rank of each sorted entry) to s_perm; token
// ids to s_ltok.  Ends with a workgroup barrier.  Every thread of the workgroup calls it.
__device__ __forceinline__ void stage_lattice_cond(const BuildParams &bp, int b, int t, int nth, float *s_raw,
                                                   float *s_logp, uint8_t *s_perm, int *s_ltok) {
  const int K = bp.K, PK = bp.P * bp.K, PKK = PK * bp.K;
  const float *e = bp.edge_logp + (size_t)b * PKK;
  const int32_t *lt = bp.lat_tok + (size_t)b * PK;
  for (int x = t; x < PKK; x += nth) s_raw[x] = e[x];
  for (int x = t; x < PK; x += nth) s_ltok[x] = lt[x];
  __syncthreads();
  for (int x = t; x < PKK; x += nth) {
    const int row = x / K, i = x - row * K;
    const float v = s_raw[x];
    int pos = 0;
    for (int j = 0; j < K; ++j) {
      const float w = s_raw[row * K + j];
      pos += (w > v || (w == v && j < i)) ? 1 : 0;
    }
    s_logp[row * K + pos] = v;
    s_perm[row * K + pos] = (uint8_t)i;
  }
  __syncthreads();
}

// Builds request b's tree.  Unless `staged` (the caller has staged the lattice with
// stage_lattice and met a workgroup barrier since), every thread of the workgroup (tid < nth)
// helps stage the lattice and meets the workgroup barrier; then the first wave alone runs the
// pops and writes the tree.  COND: the rows are parent-conditioned and already staged with
// stage_lattice_cond (s_logp sorted rows, s_perm their ranks).
template <bool COND = false>
__device__ __forceinline__ void build_request(const BuildParams &bp, int b, int tid, int nth, float *s_logp,
                                              int *s_ltok, bool staged = false, const uint8_t *s_perm = nullptr) {
  const int P = bp.P, K = bp.K, N = bp.N;
  // children are offered only at depths below this request's own position count
  const int Pb = bp.positions ? min(max(bp.positions[b], 0), P) : P;
  const gdntree_tree &out = bp.out;
  const int PK = P * K;
  if (!COND && !staged) {
    stage_lattice(bp, b, tid, nth, s_logp, s_ltok);
    __syncthreads();
  }
  if (tid >= 64) return;  // one wave builds
  const int lane = tid;
  const int root_token = bp.root_tok[b];  // loaded now, used after the pops
  // first-child log-prob of a node at depth d (children sit at lattice position d): lane d.
  // Conditioned: the first (sorted) entry and its rank of every row, row w in lane w % 64 of
  // register w / 64 (at most 16 x 16 rows).
  const float lp_first = s_logp[min(lane, P - 1) * K];
  float cf_lp[4];
  int cf_rk[4];
  if constexpr (COND) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = min(64 * j + lane, PK - 1);
      cf_lp[j] = s_logp[row * K];
      cf_rk[j] = s_perm[row * K];
    }
  }
  // the first child of row `row` (uniform): its log-prob and rank
  auto first_of = [&](int row, float &lp, int &rk) {
    const int j = row >> 6, l = row & 63;
    const float v = j == 0 ? cf_lp[0] : j == 1 ? cf_lp[1] : j == 2 ? cf_lp[2] : cf_lp[3];
    const int k = j == 0 ? cf_rk[0] : j == 1 ? cf_rk[1] : j == 2 ? cf_rk[2] : cf_rk[3];
    lp = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
    rk = __builtin_amdgcn_readlane(k, l);
  };

  // Lane l holds node l (its slot) and the one frontier candidate it offers (`has`): its
  // lowest unexpanded child rank `next`, that child's score `cand`, and, fetched ahead, the
  // log-prob `nlp` of the rank after it, so no LDS read sits between two pops.  Whether a
  // lane offers a candidate is a flag of its own: a candidate's score may be -inf (a log-prob
  // of -inf, or a finite fp64 sum that rounds to -inf in fp32) and is still a candidate.
  const double kNone = -__builtin_inf();
  int my_parent = -1, my_depth = 0, my_rank = -1, my_next = 0;
  double my_score = 0.0, cand = kNone;
  bool has = false;
  // conditioned: the rank of the child on offer and, fetched ahead with `nlp`, of the next one;
  // `byrank`: the node's children are offered in rank order (its score is -inf)
  int my_crank = 0, ncr = 0;
  bool byrank = false;
  const float *s_raw = s_logp + (COND ? bp.P * K * K : 0);  // conditioned: the unsorted rows follow
  unsigned long long my_anc = 0ull;
  // LDS index of the fetched-ahead log-prob; every lane reloads its entry after each pop
  // (one unconditional read, so the value lands straight in its register)
  int nlp_at = 0;
  if (lane == 0) {  // the root (P >= 1 and K >= 1); no children when the request has no positions
    has = Pb > 0;
    cand = 0.0 + (double)s_logp[0];  // row 0 for the conditioned rows too: position 0, the root
    nlp_at = min(1, K - 1);
    if constexpr (COND) my_crank = s_perm[0];
  }
  float nlp = s_logp[nlp_at];
  if constexpr (COND) ncr = s_perm[nlp_at];
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
    const int nx = __builtin_amdgcn_readlane(my_next, p);         // index in p's child order
    const int r = COND ? __builtin_amdgcn_readlane(my_crank, p) : nx;  // the child's rank
    const int dp = __builtin_amdgcn_readlane(my_depth, p);
    const int d = dp + 1;
    const unsigned long long a = readlane_u64(my_anc, p) | (1ull << (n - 1));
    // the new node's row of children and its first child
    const int row_n = COND ? min(d, P - 1) * K + r : min(d, P - 1);
    float first;
    int first_rk = 0;
    if constexpr (COND) {
      if (m == kNone) {  // a node scored -inf: its children tie, rank order (uniform branch)
        first = s_raw[row_n * K];
        first_rk = 0;
      } else {
        first_of(row_n, first, first_rk);
      }
    } else {
      first = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lp_first), min(d, P - 1)));
    }

    // (fetched-ahead entries are clamped, always valid: one standing past the last rank or
    // position is never used)
    if (lane == p) {  // offer p's next child
      my_next = nx + 1;
      has = nx + 1 < K;
      cand = my_score + nlpd;
      const int row_p = COND ? (dp == 0 ? 0 : dp * K + my_rank) : dp;
      nlp_at = row_p * K + min(nx + 2, K - 1);
      if constexpr (COND) my_crank = byrank ? nx + 1 : ncr;
    }
    if (n < 64) {
      if (lane == n) {
        my_parent = p; my_depth = d; my_rank = r; my_score = m; my_anc = a;
        my_next = 0;
        has = d < Pb;
        cand = m + (double)first;
        nlp_at = row_n * K + min(1, K - 1);
        if constexpr (COND) {
          my_crank = first_rk;
          byrank = m == kNone;
        }
      }
    } else {
      x_parent = p; x_depth = d; x_rank = r; x_score = m; x_anc = a;
    }
    if constexpr (COND) {
      nlp = byrank ? s_raw[nlp_at] : s_logp[nlp_at];
      ncr = s_perm[nlp_at];
    } else {
      nlp = s_logp[nlp_at];
    }
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
