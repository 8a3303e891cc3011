// Greedy acceptance plus bonus token, then the accepted-path state commit, on gfx950.
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
// One workgroup of 256 lanes owns 32 value channels j of one (layer, request, head): eight
// lanes per channel, each holding 16 (d_k = 128) or 8 (d_k = 64) entries of column j of
// the state, which is one contiguous row of the [d_v][d_k] layout.  Wave 0 of every
// workgroup walks its request's tree itself (at most 17 ballot steps over 65 slots), so
// acceptance and commit are one launch.

#include <type_traits>

#include "gdntree_internal.h"

namespace gdntree {
namespace {

template <int D, bool BF16IN>
__global__ __launch_bounds__(256) void accept_commit_kernel(CommitParams p) {
  typedef typename std::conditional<BF16IN, uint16_t, float>::type T;
  constexpr int SL = D / 32;       // workgroups (slices of 32 channels) per head
  constexpr int EPL = D / 8;       // state entries per lane
  constexpr int F4 = EPL / 4;      // float4 per lane
  __shared__ float s_k[kMaxAnc][D];
  __shared__ float s_v[kMaxAnc][32];
  __shared__ float s_a[kMaxAnc], s_b[kMaxAnc];
  __shared__ int s_path[kMaxAnc];
  __shared__ int s_tok[kMaxSlots];
  __shared__ int s_len, s_bonus;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hh = blockIdx.x / SL, js = blockIdx.x % SL;
  const int h = hh % p.H, lb = hh / p.H, b = lb % p.B, l = lb / p.B;
  const int c = tid >> 3, sub = tid & 7;
  const int j = js * 32 + c;

  // state column j, entries i = 4 * (sub + 8 m) + 0..3
  float *col = p.state + ((size_t)hh * D + j) * D;
  float4 st[F4];
#pragma unroll
  for (int m = 0; m < F4; ++m) st[m] = *reinterpret_cast<const float4 *>(col + 4 * (sub + 8 * m));

  const int n = p.n_nodes[b];
  const bool n_ok = n >= 1 && n <= p.R;
  if (wave == 0) {
    const size_t tb = (size_t)b * p.R;
    int par0 = -1, tok0 = 0, tgt0 = 0, par1 = -1, tok1 = 0, tgt1 = 0;
    if (n_ok && lane < n) { par0 = p.parent[tb + lane]; tok0 = p.token[tb + lane]; tgt0 = p.target[tb + lane]; }
    if (n_ok && lane + 64 < n) { par1 = p.parent[tb + lane + 64]; tok1 = p.token[tb + lane + 64]; tgt1 = p.target[tb + lane + 64]; }
    if (n_ok && lane < n) s_tok[lane] = tok0;
    if (n_ok && lane + 64 < n) s_tok[lane + 64] = tok1;
    int u = 0, len = 1;
    if (lane == 0) s_path[0] = 0;
    while (n_ok && len <= p.P) {
      const int tu = (u < 64) ? __builtin_amdgcn_readlane(tgt0, u) : __builtin_amdgcn_readlane(tgt1, u - 64);
      const unsigned long long m0 = __ballot(lane >= 1 && lane < n && par0 == u && tok0 == tu);
      const unsigned long long m1 = __ballot(lane + 64 < n && par1 == u && tok1 == tu);
      int cnode;
      if (m0) cnode = __ffsll((long long)m0) - 1;
      else if (m1) cnode = 64 + __ffsll((long long)m1) - 1;
      else break;
      u = cnode;
      if (lane == 0) s_path[len] = u;
      ++len;
    }
    if (lane == 0) {
      s_len = n_ok ? len : 0;
      s_bonus = (u < 64) ? __builtin_amdgcn_readlane(tgt0, u) : __builtin_amdgcn_readlane(tgt1, u - 64);
    }
  }
  __syncthreads();
  const int len = s_len;
  if (len == 0) return;  // malformed node count: nothing is written

  if (l == 0 && h == 0 && js == 0 && tid <= p.P) {
    const size_t ab = (size_t)b * (p.P + 1);
    if (tid == 0) p.acc_len[b] = len;
    p.acc_node[ab + tid] = tid < len ? s_path[tid] : -1;
    p.acc_tok[ab + tid] = tid < len - 1 ? s_tok[s_path[tid + 1]] : (tid == len - 1 ? s_bonus : -1);
  }

  // rows of the accepted path: k (all d_k), v (this slice's 32 channels), alpha, beta
  const T *gk = static_cast<const T *>(p.k);
  const T *gv = static_cast<const T *>(p.v);
  const T *ga = static_cast<const T *>(p.alpha);
  const T *gb = static_cast<const T *>(p.beta);
  const size_t rowbase = (size_t)lb * p.R;
  for (int e = tid; e < len * (D + 32); e += 256) {
    const int x = e / (D + 32), r = e % (D + 32);
    const size_t ro = ((rowbase + s_path[x]) * p.H + h) * (size_t)D;
    if (r < D) s_k[x][r] = load_elem(gk, ro + r);
    else s_v[x][r - D] = load_elem(gv, ro + js * 32 + (r - D));
  }
  for (int x = tid; x < len; x += 256) {
    const size_t gi = (rowbase + s_path[x]) * p.H + h;
    s_a[x] = load_elem(ga, gi);
    s_b[x] = load_elem(gb, gi);
  }
  __syncthreads();

  for (int x = 0; x < len; ++x) {
    float dot = 0.f;
#pragma unroll
    for (int m = 0; m < F4; ++m) {
      const float4 kk = *reinterpret_cast<const float4 *>(&s_k[x][4 * (sub + 8 * m)]);
      dot += kk.x * st[m].x + kk.y * st[m].y + kk.z * st[m].z + kk.w * st[m].w;
    }
    dot += __shfl_xor(dot, 1);
    dot += __shfl_xor(dot, 2);
    dot += __shfl_xor(dot, 4);
    const float a = s_a[x];
    const float coef = s_b[x] * (s_v[x][c] - a * dot);  // S <- a S + k (b (v - a k.S))
#pragma unroll
    for (int m = 0; m < F4; ++m) {
      const float4 kk = *reinterpret_cast<const float4 *>(&s_k[x][4 * (sub + 8 * m)]);
      st[m].x = a * st[m].x + kk.x * coef;
      st[m].y = a * st[m].y + kk.y * coef;
      st[m].z = a * st[m].z + kk.z * coef;
      st[m].w = a * st[m].w + kk.w * coef;
    }
  }
#pragma unroll
  // Non-temporal stores: the committed state is next read by the following step's verify, long
  // after this batch's other traffic, so it is written through instead of lingering dirty in
  // the caches (measured: the next verify runs 1.3-1.4 us faster, the commit no slower).
  for (int m = 0; m < F4; ++m)
    __builtin_nontemporal_store(f32x4{st[m].x, st[m].y, st[m].z, st[m].w},
                                reinterpret_cast<f32x4 *>(col + 4 * (sub + 8 * m)));
}

template <int D, bool BF16IN>
hipError_t launch_d(const CommitParams &p, hipStream_t stream) {
  const long long blocks = (long long)p.L * p.B * p.H * (D / 32);
  hipLaunchKernelGGL((accept_commit_kernel<D, BF16IN>), dim3((unsigned)blocks), dim3(256), 0,
                     stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_accept_commit(const CommitParams &p, hipStream_t stream) {
  if (p.D == 64) return p.in_bf16 ? launch_d<64, true>(p, stream) : launch_d<64, false>(p, stream);
  return p.in_bf16 ? launch_d<128, true>(p, stream) : launch_d<128, false>(p, stream);
}

}  // namespace gdntree
