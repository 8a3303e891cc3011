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
  if ((PKK & 3) == 0 && (reinterpret_cast<uintptr_t>(e) & 15) == 0) {  // whole 16-byte pieces
    const float4 *e4 = reinterpret_cast<const float4 *>(e);
    float4 *r4 = reinterpret_cast<float4 *>(s_raw);
    for (int x = t; x < PKK / 4; x += nth) r4[x] = e4[x];
  } else {
    for (int x = t; x < PKK; x += nth) s_raw[x] = e[x];
  }
  for (int x = t; x < PK; x += nth) s_ltok[x] = lt[x];
  __syncthreads();
  // one row per thread, held in registers: each entry's place is the number of entries of the
  // row that come before it (larger, or equal with a smaller rank)
  for (int row = t; row < PK; row += nth) {
    float v[kCondMaxK];
#pragma unroll
    for (int i = 0; i < kCondMaxK; ++i) v[i] = i < K ? s_raw[row * K + i] : 0.f;
#pragma unroll
    for (int i = 0; i < kCondMaxK; ++i) {
      if (i < K) {
        int pos = 0;
#pragma unroll
        for (int j = 0; j < kCondMaxK; ++j)
          pos += (j < K && (v[j] > v[i] || (v[j] == v[i] && j < i))) ? 1 : 0;
        s_logp[row * K + pos] = v[i];
        s_perm[row * K + pos] = (uint8_t)i;
      }
    }
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
  // (all four registers are read and the pick is made on scalars: no branch on j)
  auto first_of = [&](int row, float &lp, int &rk) {
    const int j = row >> 6, l = row & 63;
    int v[4], k[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      v[x] = __builtin_amdgcn_readlane(__float_as_int(cf_lp[x]), l);
      k[x] = __builtin_amdgcn_readlane(cf_rk[x], l);
    }
    const int v01 = j & 1 ? v[1] : v[0], v23 = j & 1 ? v[3] : v[2];
    const int k01 = j & 1 ? k[1] : k[0], k23 = j & 1 ? k[3] : k[2];
    lp = __int_as_float(j & 2 ? v23 : v01);
    rk = j & 2 ? k23 : k01;
  };

  // Lane l holds node l (its slot) and the one frontier candidate it offers: its lowest
  // unexpanded child rank `next`, that child's score `cand`, and, fetched ahead, the log-prob
  // `nlp` of the rank after it, so no LDS read sits between two pops.  Which lanes offer a
  // candidate is a wave mask of its own (`offer`): a candidate's score may be -inf (a log-prob
  // of -inf, or a finite fp64 sum that rounds to -inf in fp32) and is still a candidate.  `key`
  // is the candidate's score rounded to fp32 (-inf for a lane that offers none).  The pops are
  // branch-free: every lane evaluates both updates and keeps the one for its role.
  const double kNone = -__builtin_inf();
  const float kNoneF = -__builtin_inff();
  int my_parent = -1, my_depth = 0, my_rank = -1, my_next = 0;
  double my_score = 0.0, cand = kNone;
  float key = kNoneF;
  unsigned long long offer = 0ull;  // uniform: lanes that offer a candidate
  // conditioned: the rank of the child on offer and, fetched ahead with `nlp`, of the next one;
  // `byrank`: the node's children are offered in rank order (its score is -inf)
  int my_crank = 0, ncr = 0;
  bool byrank = false;
  const float *s_raw = s_logp + (COND ? bp.P * K * K : 0);  // conditioned: the unsorted rows follow
  // LDS index of the fetched-ahead log-prob; every lane reloads its entry after each pop
  // (one unconditional read, so the value lands straight in its register)
  int nlp_at = 0;
  if (lane == 0) {  // the root (P >= 1 and K >= 1); no children when the request has no positions
    cand = 0.0 + (double)s_logp[0];  // row 0 for the conditioned rows too: position 0, the root
    key = (float)cand;
    nlp_at = min(1, K - 1);
    if constexpr (COND) my_crank = s_perm[0];
  }
  if (Pb > 0) offer = 1ull;
  float nlp = s_logp[nlp_at];
  if constexpr (COND) ncr = s_perm[nlp_at];
  // next, depth and (conditioned) the offered rank of every lane, packed for one lane read
  auto pack = [&]() { return my_next | (my_depth << 8) | (my_crank << 16); };
  int my_pk = pack();
  // The 65th slot (index 64) has no lane; it is the last insertion and is kept uniformly.
  int x_parent = -1, x_depth = 0, x_rank = -1;
  double x_score = 0.0;

  int n = 1;
  while (n <= N) {
    const double nlpd = (double)nlp;  // last use of the fetched-ahead value before it is refilled
    // The winner: rounding to fp32 is monotonic, so the fp64 maximum is among the offering
    // lanes whose rounded score equals the fp32 maximum; when that lane is unique it is the
    // winner, otherwise the exact fp64 maximum is taken over those lanes (ties to the lowest
    // lane, which holds the smallest parent slot).
    const float m32 = wave_max_f32(key);
    unsigned long long hit = offer & __builtin_amdgcn_fcmpf(key, m32, 1 /* ordered equal */);
    if (hit == 0ull) break;  // the trie is exhausted
    double m;
    if (__popcll(hit) == 1) {
      m = __longlong_as_double(readlane_u64((unsigned long long)__double_as_longlong(cand), __ffsll((long long)hit) - 1));
    } else {
      const bool top = (hit >> lane) & 1ull;
      m = wave_max_f64(top ? cand : kNone);
      hit &= __builtin_amdgcn_fcmp(cand, m, 1 /* ordered equal; -inf equals -inf */);
    }
    const int p = __ffsll((long long)hit) - 1;                    // smallest parent slot
    const int pk = __builtin_amdgcn_readlane(my_pk, p);
    const int nx = pk & 0xff;                                     // index in p's child order
    const int dp = (pk >> 8) & 0xff;
    const int r = COND ? (pk >> 16) : nx;                         // the child's rank
    const int d = dp + 1;
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

    // p offers its next child; the new node n (a lane below 64) offers its first child.
    // (Fetched-ahead entries are clamped, always valid: one standing past the last rank or
    // position is never used.)
    const bool is_p = lane == p, is_n = lane == n;
    const bool p_more = nx + 1 < K, n_more = d < Pb;
    const double cand_p = my_score + nlpd;          // lane p's own score and log-prob
    const double cand_n = m + (double)first;
    const int row_p = COND ? (dp == 0 ? 0 : dp * K + my_rank) : dp;
    const int at_p = row_p * K + min(nx + 2, K - 1), at_n = row_n * K + min(1, K - 1);
    if (n < 64) {
      my_parent = is_n ? p : my_parent;
      my_depth = is_n ? d : my_depth;
      my_rank = is_n ? r : my_rank;
      my_score = is_n ? m : my_score;
    } else {
      x_parent = p; x_depth = d; x_rank = r; x_score = m;
    }
    const bool up_n = is_n && n < 64;
    cand = is_p ? cand_p : (up_n ? cand_n : cand);
    key = is_p ? (p_more ? (float)cand_p : kNoneF) : (up_n ? (n_more ? (float)cand_n : kNoneF) : key);
    my_next = is_p ? nx + 1 : (up_n ? 0 : my_next);
    nlp_at = is_p ? at_p : (up_n ? at_n : nlp_at);
    if constexpr (COND) {
      my_crank = is_p ? (byrank ? nx + 1 : ncr) : (up_n ? first_rk : my_crank);
      byrank = up_n ? (m == kNone) : byrank;
    }
    offer = p_more ? offer : (offer & ~(1ull << p));
    if (n < 64 && n_more) offer |= 1ull << n;
    my_pk = pack();
    if constexpr (COND) {
      nlp = (byrank ? s_raw : s_logp)[nlp_at];
      ncr = s_perm[nlp_at];
    } else {
      nlp = s_logp[nlp_at];
    }
    ++n;
  }

  // Ancestor masks after the build, by pointer jumping over the parent links: bit t-1 of node
  // t, then each round ORs in the mask of the node 2^i links up (depth <= 16: five rounds).
  unsigned long long my_anc = (lane >= 1 && lane < n) ? (1ull << (lane - 1)) : 0ull;
  int up = (lane >= 1 && lane < n) ? my_parent : 0;
#pragma unroll
  for (int it = 0; it < 5; ++it) {
    const unsigned lo = (unsigned)__builtin_amdgcn_ds_bpermute(up << 2, (int)(unsigned)my_anc);
    const unsigned hi = (unsigned)__builtin_amdgcn_ds_bpermute(up << 2, (int)(unsigned)(my_anc >> 32));
    my_anc |= ((unsigned long long)hi << 32) | lo;
    up = __builtin_amdgcn_ds_bpermute(up << 2, up);
  }
  const unsigned long long x_anc = n == 65 ? (readlane_u64(my_anc, x_parent) | (1ull << 63)) : 0ull;

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
