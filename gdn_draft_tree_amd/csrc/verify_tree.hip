// Tree verify for Gated-DeltaNet layers on gfx950.
//
// What is computed (SpecPilot summary, Prerequisites > hybrid recurrent architecture):
// for every node t of a request's draft tree, with S_p the state of t's parent (the
// committed state S0 for the root),
//     S_t = a_t (I - b_t k_t k_t^T) S_p + b_t k_t v_t^T,      o_t = S_t^T q_t.
// The pages recompute states along root paths instead of snapshotting every node and name
// a WY-form kernel for it (Technical novelty).  This kernel never forms any node state.
//
// Tree form of the WY / UT transform.  Let anc(t) be the ancestors of t (root included),
// g_t = prod of a over root..t, and r(t,s) = g_t / g_s for s an ancestor-or-self of t.
// Writing S_t = g_t S0 + sum_{s in anc(t) + t} r(t,s) k_s u_s^T, the pseudo-values u solve
// the tree-triangular system
//     u_t + sum_{s in anc(t)} Lm[t,s] u_s = b_t (v_t - g_t S0^T k_t),
//     Lm[t,s] = b_t r(t,s) (k_t . k_s),
// and o_t = g_t S0^T q_t + sum_{s in anc(t)+t} Mm[t,s] u_s with Mm[t,s] = r(t,s)(q_t . k_s).
// With Wm = Mm (I + Lm)^-1 (same ancestor sparsity) this collapses to
//     o_t = S0^T qe_t + sum_s W1[t,s] v_s,
//     qe_t = g_t q_t - sum_s W2[t,s] k_s,   W1[t,s] = Wm[t,s] b_s,   W2 = W1[t,s] g_s,
// so S0 (the only large operand, d_k x d_v fp32) is touched by ONE dense product
// [qe_t]^T S0 over all nodes.  That product runs on bf16 MFMA with S0 and qe split into
// hi + lo bf16 parts (hi*hi + lo*hi + hi*lo; the dropped lo*lo term is ~2^-16 relative),
// the exact-split idea the pages mention for their fp32 state.  Everything that depends on
// the tree (Gram entries, gates, the ancestor-restricted solve) is O(nodes * depth) work.
//
// Work decomposition: one workgroup per (layer, request, head) and slice of d_v rows; each
// wave owns 32 value channels j (two 16-row MFMA tiles of S0^T) for all nodes.  S0^T rows
// are contiguous in the [d_v][d_k] state layout, so each lane loads its MFMA A-operand
// fragments straight from HBM, at kernel entry, while the tree prologue runs.

#include "gdntree_internal.h"

namespace gdntree {
namespace {

constexpr int kA = kMaxAnc;  // 17 ancestor slots (depth 0..16)

template <bool BF16IN>
struct InT;
template <>
struct InT<true> { typedef uint16_t T; static constexpr int kPad = 8; };
template <>
struct InT<false> { typedef float T; static constexpr int kPad = 4; };

template <int D, bool BF16IN, int NT>
struct VerifySmem {
  typedef typename InT<BF16IN>::T T;
  static constexpr int NP = 16 * NT;                  // padded node rows
  static constexpr int RS = D + InT<BF16IN>::kPad;    // K/Q/V row stride (16 B pad)
  static constexpr int QS = D + 8;                    // qe hi/lo row stride (bf16)
  alignas(16) T k[NP * RS];
  alignas(16) T q[NP * RS];                           // bf16 input: reused as qe_hi
  alignas(16) T v[BF16IN ? NP * D : 4];               // fp32 input reads v from memory
  alignas(16) uint16_t qhi[BF16IN ? 8 : NP * QS];
  alignas(16) uint16_t qlo[NP * QS];
  alignas(16) float lc[NP * kA];                      // k.k Gram -> Lm
  alignas(16) float mc[NP * kA];                      // q.k Gram -> Mm
  alignas(16) float wc[NP * kA];                      // Wm
  float alpha[NP], beta[NP], gamma[NP];
  int parent[NP];
  int8_t depth[NP];
  int8_t anc[NP * kA];                                // ancestor slot at each depth
  int bad;
};

// 8 consecutive elements of an LDS row as one MFMA operand (bf16 input: exact).
__device__ __forceinline__ bf16x8 lds_frag(const uint16_t *row) {
  const uint4 u = *reinterpret_cast<const uint4 *>(row);
  return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ void split8(const float *x, bf16x8 &hi, bf16x8 &lo) {
  u16x8 h, l;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint16_t hb = f32_to_bf16_bits(x[i]);
    h[i] = hb;
    l[i] = f32_to_bf16_bits(x[i] - bf16_bits_to_f32(hb));
  }
  hi = __builtin_bit_cast(bf16x8, h);
  lo = __builtin_bit_cast(bf16x8, l);
}

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Gram tile product for rows ra (of A) and rb (of B), 8 columns per lane per k-step.
template <int D, bool BF16IN>
__device__ __forceinline__ f32x4 gram_tile(const typename InT<BF16IN>::T *A, const typename InT<BF16IN>::T *Bm,
                                           int rs, int ra, int rb, int kofs) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    const int col = 32 * ks + kofs;
    if constexpr (BF16IN) {
      acc = mfma(lds_frag(A + ra * rs + col), lds_frag(Bm + rb * rs + col), acc);
    } else {
      float xa[8], xb[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) { xa[i] = A[ra * rs + col + i]; xb[i] = Bm[rb * rs + col + i]; }
      bf16x8 ah, al, bh, bl;
      split8(xa, ah, al);
      split8(xb, bh, bl);
      acc = mfma(ah, bh, acc);
      acc = mfma(al, bh, acc);
      acc = mfma(ah, bl, acc);
    }
  }
  return acc;
}

template <int D, bool BF16IN, int NT>
__global__ __launch_bounds__(256) void verify_kernel(VerifyParams p) {
  typedef VerifySmem<D, BF16IN, NT> SM;
  typedef typename SM::T T;
  constexpr int NP = SM::NP, RS = SM::RS, QS = SM::QS;
  constexpr int KS = D / 32;        // MFMA k-steps over d_k
  constexpr int CH = 16 / sizeof(T);  // elements per 16-byte chunk
  __shared__ SM s;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nthr = blockDim.x, W = nthr >> 6;
  const int S = D / (32 * W);  // d_v slices per head
  int hh, js;
  if (S == 1) {
    hh = blockIdx.x;
    js = 0;
  } else {  // keep a head's slices on one XCD (workgroups are dealt round-robin to 8 XCDs)
    const int xcd = blockIdx.x & 7, loc = blockIdx.x >> 3;
    js = loc % S;
    hh = (loc / S) * 8 + xcd;
  }
  const int HT = p.L * p.B * p.H;
  if (hh >= HT) return;
  const int h = hh % p.H, lb = hh / p.H, b = lb % p.B;
  const int n = p.n_nodes[b];
  if (n < 1 || n > p.R) return;  // malformed count: nothing is written

  const size_t rowbase = (size_t)lb * p.R;  // (l*B + b) * R
  const T *gq = static_cast<const T *>(p.q);
  const T *gk = static_cast<const T *>(p.k);
  const T *gv = static_cast<const T *>(p.v);
  const T *ga = static_cast<const T *>(p.alpha);
  const T *gb = static_cast<const T *>(p.beta);
  auto row_off = [&](int t) -> size_t { return ((rowbase + t) * p.H + h) * (size_t)D; };

  // ---- 0. this wave's S0^T operand fragments (rows j, 8 consecutive i per lane) --------
  const int j0 = js * 32 * W + wave * 32;
  const float *sbase = p.state + (size_t)hh * D * D;
  float4 sraw[2][KS][2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const float4 *ptr = reinterpret_cast<const float4 *>(
          sbase + (size_t)(j0 + 16 * mt + (lane & 15)) * D + 32 * ks + 8 * (lane >> 4));
      sraw[mt][ks][0] = ptr[0];
      sraw[mt][ks][1] = ptr[1];
    }

  // ---- 1. tree metadata, gates and the K / Q (/ V) rows of the n used slots -----------
  if (tid == 0) s.bad = 0;
  for (int t = tid; t < n; t += nthr) {
    s.parent[t] = p.parent[(size_t)b * p.R + t];
    const size_t gi = (rowbase + t) * p.H + h;
    s.alpha[t] = load_elem(ga, gi);
    s.beta[t] = load_elem(gb, gi);
  }
  {
    constexpr int CPR = D / CH;  // chunks per row
    const int nmat = BF16IN ? 3 : 2;
    const int total = nmat * n * CPR;
    for (int c = tid; c < total; c += nthr) {
      const int m = c / (n * CPR), rem = c % (n * CPR), t = rem / CPR, cc = rem % CPR;
      const T *src = (m == 0 ? gk : m == 1 ? gq : gv) + row_off(t) + cc * CH;
      const uint4 val = *reinterpret_cast<const uint4 *>(src);
      T *dst = (m == 0) ? s.k + t * RS + cc * CH : (m == 1) ? s.q + t * RS + cc * CH : s.v + t * D + cc * CH;
      *reinterpret_cast<uint4 *>(dst) = val;
    }
  }
  __syncthreads();

  // depth, ancestor table and path gate of each node (walks parent links; checks them)
  for (int t = tid; t < n; t += nthr) {
    int x = t, dep = 0;
    bool ok = true;
    while (x > 0) {
      const int px = s.parent[x];
      if (px < 0 || px >= x || ++dep > kMaxP) { ok = false; break; }
      x = px;
    }
    if (!ok) {
      s.bad = 1;
    } else {
      s.depth[t] = (int8_t)dep;
      x = t;
      for (int e = dep; e >= 0; --e) {
        s.anc[t * kA + e] = (int8_t)x;
        if (e > 0) x = s.parent[x];
      }
      float g = 1.f;
      for (int e = 0; e <= dep; ++e) g *= s.alpha[s.anc[t * kA + e]];
      s.gamma[t] = g;
    }
  }
  __syncthreads();

  const int jw0 = js * 32 * W;  // this workgroup's first value channel
  if (s.bad) {
    const int span = 32 * W;
    for (int c = tid; c < n * span; c += nthr) {
      const int t = c / span, j = jw0 + c % span;
      const size_t oi = row_off(t) + j;
      if (p.out_bf16) static_cast<uint16_t *>(p.o)[oi] = 0x7fc0;
      else static_cast<float *>(p.o)[oi] = __builtin_nanf("");
    }
    return;
  }

  // ---- 2. Gram entries k_t.k_s and q_t.k_s for s ancestor-or-self of t (MFMA) ---------
  {
    constexpr int NPAIR = NT * (NT + 1) / 2;
    for (int pi = wave; pi < 2 * NPAIR; pi += W) {
      const int part = pi >= NPAIR;  // 0: k.k, 1: q.k
      const int qi = part ? pi - NPAIR : pi;
      int mt = 0;
      while ((mt + 1) * (mt + 2) / 2 <= qi) ++mt;
      const int nt = qi - mt * (mt + 1) / 2;
      if (16 * mt >= n) continue;
      const f32x4 g = gram_tile<D, BF16IN>(part ? s.q : s.k, s.k, RS, 16 * mt + (lane & 15),
                                           16 * nt + (lane & 15), 8 * (lane >> 4));
      const int sn = 16 * nt + (lane & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * mt + 4 * (lane >> 4) + r;
        if (t < n && sn <= t) {
          const int e = s.depth[sn];
          if (e <= s.depth[t] && s.anc[t * kA + e] == sn) (part ? s.mc : s.lc)[t * kA + e] = g[r];
        }
      }
    }
  }
  __syncthreads();

  // ---- 3. gate ratios: Lm and Mm rows --------------------------------------------------
  for (int t = tid; t < n; t += nthr) {
    const int dt = s.depth[t];
    const float bt = s.beta[t];
    float rho = 1.f;  // g_t / g_{anc at depth e}
    for (int e = dt; e >= 0; --e) {
      s.mc[t * kA + e] *= rho;
      if (e < dt) s.lc[t * kA + e] *= bt * rho;
      rho *= s.alpha[s.anc[t * kA + e]];
    }
  }
  __syncthreads();

  // Wm row t solves Wm (I + Lm) = Mm over t's path, deepest ancestor first.
  for (int t = tid; t < n; t += nthr) {
    const int dt = s.depth[t];
    float w[kA];
#pragma unroll
    for (int e = kA - 1; e >= 0; --e) {
      float acc = 0.f;
      if (e <= dt) {
        acc = s.mc[t * kA + e];
#pragma unroll
        for (int e2 = e + 1; e2 < kA; ++e2)
          if (e2 <= dt) acc -= w[e2] * s.lc[s.anc[t * kA + e2] * kA + e];
      }
      w[e] = acc;
    }
#pragma unroll
    for (int e = 0; e < kA; ++e)
      if (e <= dt) s.wc[t * kA + e] = w[e];
  }
  __syncthreads();

  // ---- 4. effective queries qe_t = g_t q_t - sum_s W2[t,s] k_s, split hi/lo (bf16) ------
  {
    uint16_t *qhi = BF16IN ? reinterpret_cast<uint16_t *>(s.q) : s.qhi;
    constexpr int C8 = D / 8;
    for (int it = tid; it < NP * C8; it += nthr) {
      const int t = it / C8, c = it % C8;
      float x[8];
      if (t < n) {
        const float g = s.gamma[t];
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = g * load_elem(s.q, (size_t)t * RS + 8 * c + i);
        const int dt = s.depth[t];
        for (int e = 0; e <= dt; ++e) {
          const int sn = s.anc[t * kA + e];
          const float w2 = s.wc[t * kA + e] * s.beta[sn] * s.gamma[sn];
#pragma unroll
          for (int i = 0; i < 8; ++i) x[i] -= w2 * load_elem(s.k, (size_t)sn * RS + 8 * c + i);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = 0.f;
      }
      bf16x8 hi, lo;
      split8(x, hi, lo);
      *reinterpret_cast<bf16x8 *>(qhi + t * QS + 8 * c) = hi;
      *reinterpret_cast<bf16x8 *>(s.qlo + t * QS + 8 * c) = lo;
    }
  }
  __syncthreads();

  // ---- 5-7. o^T = S0^T [qe] + V^T W1^T, node tile by node tile -------------------------
  bf16x8 ahi[2][KS], alo[2][KS];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const float x[8] = {sraw[mt][ks][0].x, sraw[mt][ks][0].y, sraw[mt][ks][0].z, sraw[mt][ks][0].w,
                          sraw[mt][ks][1].x, sraw[mt][ks][1].y, sraw[mt][ks][1].z, sraw[mt][ks][1].w};
      split8(x, ahi[mt][ks], alo[mt][ks]);
    }
  const uint16_t *qhi = BF16IN ? reinterpret_cast<const uint16_t *>(s.q) : s.qhi;
  const int ntiles = (n + 15) / 16;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    if (nt >= ntiles) break;
    const int t = 16 * nt + (lane & 15);
    const int jl = j0 + 4 * (lane >> 4);  // + 16*mt + r
    f32x4 acc0[2], acc1[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      acc0[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      acc1[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // V^T W1^T on the vector ALUs (ancestor-sparse)
    if (t < n) {
      const int dt = s.depth[t];
      for (int e = 0; e <= dt; ++e) {
        const int sn = s.anc[t * kA + e];
        const float w1 = s.wc[t * kA + e] * s.beta[sn];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          float vv[4];
          if constexpr (BF16IN) {
            const uint2 u = *reinterpret_cast<const uint2 *>(s.v + sn * D + jl + 16 * mt);
            vv[0] = bf16_bits_to_f32(u.x & 0xffff); vv[1] = bf16_bits_to_f32(u.x >> 16);
            vv[2] = bf16_bits_to_f32(u.y & 0xffff); vv[3] = bf16_bits_to_f32(u.y >> 16);
          } else {
            const float4 u = *reinterpret_cast<const float4 *>(gv + row_off(sn) + jl + 16 * mt);
            vv[0] = u.x; vv[1] = u.y; vv[2] = u.z; vv[3] = u.w;
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) acc0[mt][r] += w1 * vv[r];
        }
      }
    }
    // S0^T qe on MFMA: hi*hi into acc0, the two cross terms into acc1
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int col = 32 * ks + 8 * (lane >> 4);
      const bf16x8 bhi = lds_frag(qhi + t * QS + col);
      const bf16x8 blo = lds_frag(s.qlo + t * QS + col);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        acc0[mt] = mfma(ahi[mt][ks], bhi, acc0[mt]);
        acc1[mt] = mfma(alo[mt][ks], bhi, acc1[mt]);
        acc1[mt] = mfma(ahi[mt][ks], blo, acc1[mt]);
      }
    }
    if (t < n) {
      const size_t ob = row_off(t);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const int j = jl + 16 * mt;
        const float o0 = acc0[mt][0] + acc1[mt][0], o1 = acc0[mt][1] + acc1[mt][1];
        const float o2 = acc0[mt][2] + acc1[mt][2], o3 = acc0[mt][3] + acc1[mt][3];
        if (p.out_bf16) {
          uint2 u;
          u.x = (uint32_t)f32_to_bf16_bits(o0) | ((uint32_t)f32_to_bf16_bits(o1) << 16);
          u.y = (uint32_t)f32_to_bf16_bits(o2) | ((uint32_t)f32_to_bf16_bits(o3) << 16);
          *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(p.o) + ob + j) = u;
        } else {
          *reinterpret_cast<float4 *>(static_cast<float *>(p.o) + ob + j) = make_float4(o0, o1, o2, o3);
        }
      }
    }
  }
}

template <int D, bool BF16IN, int NT>
hipError_t launch_one(const VerifyParams &p, hipStream_t stream) {
  const int HT = p.L * p.B * p.H;
  int W = D / 32;  // waves per workgroup (one per 32 value channels)
  if (HT < 256) W = (HT >= 128 && D / 64 >= 1) ? D / 64 : 1;
  const int S = D / (32 * W);
  const long long blocks = (S == 1) ? HT : (long long)((HT + 7) / 8) * 8 * S;
  hipLaunchKernelGGL((verify_kernel<D, BF16IN, NT>), dim3((unsigned)blocks), dim3(64 * W), 0,
                     stream, p);
  return hipGetLastError();
}

template <int D, bool BF16IN>
hipError_t launch_nt(const VerifyParams &p, hipStream_t stream) {
  switch ((p.R + 15) / 16) {
    case 1: return launch_one<D, BF16IN, 1>(p, stream);
    case 2: return launch_one<D, BF16IN, 2>(p, stream);
    case 3: return launch_one<D, BF16IN, 3>(p, stream);
    case 4: return launch_one<D, BF16IN, 4>(p, stream);
    default: return launch_one<D, BF16IN, 5>(p, stream);
  }
}

}  // namespace

hipError_t launch_verify(const VerifyParams &p, hipStream_t stream) {
  if (p.D == 64) return p.in_bf16 ? launch_nt<64, true>(p, stream) : launch_nt<64, false>(p, stream);
  return p.in_bf16 ? launch_nt<128, true>(p, stream) : launch_nt<128, false>(p, stream);
}

}  // namespace gdntree
