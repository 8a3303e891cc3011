// Greedy acceptance plus bonus token, and the accepted-path state commit, on gfx950 (device
// code shared by the acceptance and commit kernels and the fused commit + next-build kernel).
//
// Acceptance (SpecPilot summary, Prerequisites > speculative decoding and > draft-tree
// verification): from the root, repeatedly step to the child whose token equals the
// target's argmax at the current node (smallest slot on a tie); tau = steps + 1 and the
// bonus token is the target's argmax at the last accepted node.
// Commit (same page, Prerequisites > hybrid recurrent architecture: states are recomputed
// along root paths, not snapshotted): the request's state becomes the state of the deepest
// accepted node, recomputed from the committed state through the tau accepted rows with
// the gated delta rule and written back in place.
//
// Commit kernel: one workgroup of 256 lanes per (layer, request, head), in the [d_k][d_v]
// state layout: lane (w, l) of the first 2 d lanes owns value channel j = 32 w + (l & 31) and
// the half l >> 5 of its column (d/2 entries), so each load or store instruction moves two
// 128-byte runs of consecutive channels, and the column's dot product k . S_j is the sum of
// the two halves, one lane-exchange away.  Either wave 0 walks its request's tree itself (at
// most 17 ballot steps over 65 slots), so that acceptance and commit are one launch, or the
// workgroup takes the accepted path that the acceptance kernel (one wave per request) wrote
// before.
//
// The tau rank-1 updates S_x = a_x S_{x-1} + k_x c_x^T, c_x = b_x (v_x - a_x S_{x-1}^T k_x), are
// applied in the unrolled (WY) form: with G_x the product of the gates a_0..a_x and
// R(x, y) = G_x / G_y the product of a_{y+1}..a_x,
//     S_{x-1}^T k_x = G_{x-1} S_0^T k_x + sum_{y < x} R(x-1, y) (k_x . k_y) c_y,
//     S_tau-1 = G_{tau-1} S_0 + sum_y R(tau-1, y) k_y c_y^T,
// so the tau dot products with the committed state are independent (no step waits on the
// previous one's update), the Gram entries k_x . k_y are shared by the workgroup, and only a
// scalar recurrence over the c_x of each column is sequential.

#pragma once

#include <type_traits>

#include "gdntree_internal.h"

namespace gdntree {

// What one wave holds of a request's tree for the acceptance walk: lane l has slots l and
// l + 64 (parent, token, target argmax), loaded for every slot below R.
struct WalkRegs {
  int n, par0, tok0, tgt0, par1, tok1, tgt1;
};

__device__ __forceinline__ WalkRegs walk_load(const int32_t *parent, const int32_t *token, const int32_t *target,
                                              const int32_t *n_nodes, int R, int b, int lane) {
  WalkRegs w{n_nodes[b], -1, 0, 0, -1, 0, 0};
  const size_t tb = (size_t)b * R;
  if (lane < R) { w.par0 = parent[tb + lane]; w.tok0 = token[tb + lane]; w.tgt0 = target[tb + lane]; }
  if (lane + 64 < R) { w.par1 = parent[tb + lane + 64]; w.tok1 = token[tb + lane + 64]; w.tgt1 = target[tb + lane + 64]; }
  return w;
}

// The acceptance walk of one request by one wave, from the values walk_load fetched:
// s_path[0..len) = the accepted slots from the root, s_tok = the tokens of the used slots,
// *s_len = tau (0 for a node count outside [1, R]), *s_bonus = the target's argmax at the last
// accepted node.  Lane 0 writes the scalars and the path.
__device__ __forceinline__ void walk_run(const WalkRegs &w, int R, int P, int lane, int *s_path, int *s_tok,
                                         int *s_len, int *s_bonus) {
  const int n = w.n;
  const bool n_ok = n >= 1 && n <= R;
  if (n_ok && lane < n) s_tok[lane] = w.tok0;
  if (n_ok && lane + 64 < n) s_tok[lane + 64] = w.tok1;
  int u = 0, len = 1;
  if (lane == 0) s_path[0] = 0;
  while (n_ok && len <= P) {
    const int tu = (u < 64) ? __builtin_amdgcn_readlane(w.tgt0, u) : __builtin_amdgcn_readlane(w.tgt1, u - 64);
    const unsigned long long m0 = __ballot(lane >= 1 && lane < n && w.par0 == u && w.tok0 == tu);
    const unsigned long long m1 = __ballot(lane + 64 < n && w.par1 == u && w.tok1 == tu);
    int cnode;
    if (m0) cnode = __ffsll((long long)m0) - 1;
    else if (m1) cnode = 64 + __ffsll((long long)m1) - 1;
    else break;
    u = cnode;
    if (lane == 0) s_path[len] = u;
    ++len;
  }
  if (lane == 0) {
    *s_len = n_ok ? len : 0;
    *s_bonus = (u < 64) ? __builtin_amdgcn_readlane(w.tgt0, u) : __builtin_amdgcn_readlane(w.tgt1, u - 64);
  }
}

// The acceptance walk of request b by one wave (walk_load, then walk_run).
__device__ __forceinline__ void accept_walk(const CommitParams &p, int b, int lane, int *s_path,
                                            int *s_tok, int *s_len, int *s_bonus) {
  const WalkRegs w = walk_load(p.parent, p.token, p.target, p.n_nodes, p.R, b, lane);
  walk_run(w, p.R, p.P, lane, s_path, s_tok, s_len, s_bonus);
}

// Lanes t = 0..P write request b's acceptance result.
__device__ __forceinline__ void write_acceptance(const CommitParams &p, int b, int t, int len,
                                                 const int *s_path, const int *s_tok, int bonus) {
  const size_t ab = (size_t)b * (p.P + 1);
  if (t == 0) p.acc_len[b] = len;
  p.acc_node[ab + t] = t < len ? s_path[t] : -1;
  p.acc_tok[ab + t] = t < len - 1 ? s_tok[s_path[t + 1]] : (t == len - 1 ? bonus : -1);
}

// Register budget of the commit kernels: four waves per SIMD, so that four workgroups fit a
// CU and a batch of 32 requests x 32 heads is resident at once (a few spilled registers cost
// less than a second round of workgroups).
constexpr int kCommitWavesPerEU = 4;

template <int D>
struct CommitSmem {
  float k[kMaxAnc][D];
  float v[kMaxAnc][D];
  float a[kMaxAnc], b[kMaxAnc];
  float kk[kMaxAnc][kMaxAnc];  // Gram entries k_x . k_y of the path rows, y < x
  int path[kMaxAnc];
  int tok[kMaxSlots];
  int len, bonus, bad;
};

// Where a commit workgroup takes its request's accepted path from.
enum CommitPath {
  kPathGiven = 0,      // read from acc_len / acc_node and checked (tau in [1, P+1], slot 0
                       // first, each next slot a child of the previous one within the node
                       // count; a path that fails leaves the request's state untouched)
  kWalkAndWrite = 1,   // wave 0 walks the tree; the (0, 0) workgroup of each request writes
                       // the acceptance
  kWalk = 2,           // wave 0 walks the tree; the acceptance is written elsewhere
};

// Commit of work unit `hh` (one (layer, request, head)) by the 256 threads of a workgroup.
template <int D, bool BF16IN, int PATH>
__device__ __forceinline__ void commit_unit(const CommitParams &p, int hh, int tid, CommitSmem<D> &sm) {
  typedef typename std::conditional<BF16IN, uint16_t, float>::type T;
  constexpr int EPL = D / 2;       // state entries per lane: half a column
  static_assert(2 * D <= 256, "one lane per half column");
  float(&s_k)[kMaxAnc][D] = sm.k;
  float(&s_v)[kMaxAnc][D] = sm.v;
  float *s_a = sm.a, *s_b = sm.b;
  int *s_path = sm.path, *s_tok = sm.tok;
  int &s_len = sm.len, &s_bonus = sm.bonus, &s_bad = sm.bad;

  const int lane = tid & 63, wave = tid >> 6;
  const int h = hh % p.H, lb = hh / p.H, b = lb % p.B, l = lb / p.B;
  const bool act = tid < 2 * D;
  const int j = 32 * wave + (lane & 31), i0 = (lane >> 5) * EPL;

  // entries i0 .. i0 + EPL - 1 of column j: S[i][j] at i * D + j
  float *S = p.state + (size_t)hh * D * D;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(S, 0, D * D * 4, 0x00020000);
  const int voff = (i0 * D + j) * 4;
  float st[EPL];
  if (act) {
#pragma unroll
    for (int m = 0; m < EPL; ++m) st[m] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, voff, m * D * 4, 0));
  }

  if constexpr (PATH != kPathGiven) {
    if (wave == 0) accept_walk(p, b, lane, s_path, s_tok, &s_len, &s_bonus);
    __syncthreads();
  } else {
    const int n = p.n_nodes[b];
    const int len0 = p.acc_len[b];
    const bool ok0 = n >= 1 && n <= p.R && len0 >= 1 && len0 <= p.P + 1;
    if (tid == 0) s_bad = ok0 ? 0 : 1;
    if (ok0 && tid < len0) s_path[tid] = p.acc_node[(size_t)b * (p.P + 1) + tid];
    __syncthreads();
    if (ok0 && tid < len0) {
      const int x = s_path[tid];
      const bool ok = tid == 0 ? x == 0 : (x >= 1 && x < n && p.parent[(size_t)b * p.R + x] == s_path[tid - 1]);
      if (!ok) s_bad = 1;
    }
    __syncthreads();
    if (tid == 0) s_len = s_bad ? 0 : len0;
    __syncthreads();
  }
  const int len = s_len;
  if (len == 0) return;  // malformed node count or path: nothing is written

  if constexpr (PATH == kWalkAndWrite) {
    if (l == 0 && h == 0 && tid <= p.P) write_acceptance(p, b, tid, len, s_path, s_tok, s_bonus);
  }

  // rows of the accepted path: k and v (all channels), alpha, beta
  const T *gk = static_cast<const T *>(p.k);
  const T *gv = static_cast<const T *>(p.v);
  const T *ga = static_cast<const T *>(p.alpha);
  const T *gb = static_cast<const T *>(p.beta);
  const size_t rowbase = (size_t)lb * p.R;
  for (int e = tid; e < len * 2 * D; e += 256) {
    const int x = e / (2 * D), r = e % (2 * D);
    const size_t ro = ((rowbase + s_path[x]) * p.H + h) * (size_t)D;
    if (r < D) s_k[x][r] = load_elem(gk, ro + r);
    else s_v[x][r - D] = load_elem(gv, ro + (r - D));
  }
  for (int x = tid; x < len; x += 256) {
    const size_t gi = (rowbase + s_path[x]) * p.H + h;
    s_a[x] = load_elem(ga, gi);
    s_b[x] = load_elem(gb, gi);
  }
  __syncthreads();
  // the Gram entries of the path rows, y < x, by every thread (fp32, summed in order)
  for (int e = tid; e < kMaxAnc * kMaxAnc; e += 256) {
    const int x = e / kMaxAnc, y = e % kMaxAnc;
    if (y < x && x < len) {
      float g = 0.f;
#pragma unroll 8
      for (int i = 0; i < D; ++i) g = fmaf(s_k[x][i], s_k[y][i], g);
      sm.kk[x][y] = g;
    }
  }
  __syncthreads();
  if (!act) return;

  // d_x = k_x . S_0[:, j] for every path row: this lane's half, then the other half
  float d[kMaxAnc];
#pragma unroll
  for (int x = 0; x < kMaxAnc; ++x) {
    d[x] = 0.f;
    if (x < len) {
      float d4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < EPL; m += 4) {
        const float4 kk = *reinterpret_cast<const float4 *>(&s_k[x][i0 + m]);
        d4[0] = fmaf(kk.x, st[m], d4[0]);
        d4[1] = fmaf(kk.y, st[m + 1], d4[1]);
        d4[2] = fmaf(kk.z, st[m + 2], d4[2]);
        d4[3] = fmaf(kk.w, st[m + 3], d4[3]);
      }
      d[x] = (d4[0] + d4[1]) + (d4[2] + d4[3]);
    }
  }
#pragma unroll
  for (int x = 0; x < kMaxAnc; ++x)
    if (x < len) d[x] += __shfl_xor(d[x], 32);  // the other half of column j
  // c_x, in path order; G = G_{x-1}
  float c[kMaxAnc];
  float G = 1.f;
#pragma unroll
  for (int x = 0; x < kMaxAnc; ++x) {
    c[x] = 0.f;
    if (x < len) {
      float ks = G * d[x];  // S_{x-1}^T k_x, channel j
      float r = 1.f;        // R(x-1, y), y from x-1 down
#pragma unroll
      for (int y = kMaxAnc - 1; y >= 0; --y) {
        if (y < x) {
          ks = fmaf(r * sm.kk[x][y], c[y], ks);
          r *= s_a[y];
        }
      }
      const float a = s_a[x];
      c[x] = s_b[x] * (s_v[x][j] - a * ks);
      G *= a;
    }
  }
  // S_tau-1[:, j] = G_{tau-1} S_0[:, j] + sum_y R(tau-1, y) k_y c_y; the coefficients from the last
  // row back, R(tau-1, tau-1) = 1
  float r = 1.f;
#pragma unroll
  for (int m = 0; m < EPL; ++m) st[m] *= G;
#pragma unroll
  for (int y = kMaxAnc - 1; y >= 0; --y) {
    if (y < len) {
      const float coef = r * c[y];
#pragma unroll
      for (int m = 0; m < EPL; m += 4) {
        const float4 kk = *reinterpret_cast<const float4 *>(&s_k[y][i0 + m]);
        st[m] = fmaf(kk.x, coef, st[m]);
        st[m + 1] = fmaf(kk.y, coef, st[m + 1]);
        st[m + 2] = fmaf(kk.z, coef, st[m + 2]);
        st[m + 3] = fmaf(kk.w, coef, st[m + 3]);
      }
      r *= s_a[y];
    }
  }
  // Non-temporal stores: the committed state is next read by the following step's verify, long
  // after this batch's other traffic, so it is written through instead of lingering dirty in
  // the caches.
#pragma unroll
  for (int m = 0; m < EPL; ++m) __builtin_nontemporal_store(st[m], S + (size_t)(i0 + m) * D + j);
}

}  // namespace gdntree
