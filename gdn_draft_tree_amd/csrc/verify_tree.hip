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
//     qe_t = g_t q_t - sum_s W2[t,s] k_s,   W1[t,s] = Wm[t,s] b_s,   W2[t,s] = W1[t,s] g_s,
// so S0 (the only large operand, d_k x d_v fp32) is touched by ONE dense product
// [qe_t]^T S0 over all nodes.  That product runs on bf16 MFMA with S0 and qe split into
// hi + lo bf16 parts (hi*hi + lo*hi + hi*lo; the dropped lo*lo term is ~2^-16 relative),
// the exact-split idea the pages mention for their fp32 state.  Everything that depends on
// the tree (Gram entries, gates, the ancestor-restricted solve) is O(nodes * depth) work.
//
// Work decomposition: one workgroup per (layer, request, head) and slice of d_v rows; each
// wave owns 32 value channels j (two 16-row MFMA tiles of S0^T) for all nodes.  All three
// dense contractions run on MFMA: the Gram entries k_t.k_s and q_t.k_s; the effective
// queries [qe]^T = g [q]^T - K^T W2^T; and o^T = S0^T [qe] + V^T W1^T.  W1 and W2 are
// ancestor-masked node x node matrices, stored densely (hi + lo bf16) in LDS for the
// product; the O(nodes * depth) solve that produces them runs one thread per node.  S0^T
// rows are contiguous in the [d_v][d_k] state layout, so each lane loads its S0^T operand
// fragments straight from HBM at kernel entry, together with its K^T and V^T fragments
// (gathered along the node axis), while the tree prologue runs.  Ancestor sets come from
// the tree's ancestor bitmasks (depth = popcount), so no thread walks parent links.  LDS
// holds only the used rows (under 80 KiB at N = 64), so two workgroups share a CU.

#include "gdntree_internal.h"

namespace gdntree {
namespace {

constexpr int kA = kMaxAnc;  // 17 ancestor depths (0..16)
constexpr int kAR = 20;      // padded compact row (five 16-byte vectors)

template <bool BF16IN>
struct InT;
template <>
struct InT<true> { typedef uint16_t T; static constexpr int kPad = 8; };
template <>
struct InT<false> { typedef float T; static constexpr int kPad = 4; };

template <int D, bool BF16IN, int NT>
struct VerifySmem {
  typedef typename InT<BF16IN>::T T;
  static constexpr int RM = (16 * NT < kMaxSlots) ? 16 * NT : kMaxSlots;  // rows held
  static constexpr int RS = D + InT<BF16IN>::kPad;  // K/Q row stride (16 B pad)
  static constexpr int QS = D + 8;                  // qe hi/lo row stride (bf16)
  static constexpr int SP = (16 * NT + 31) / 32 * 32;  // node axis padded for MFMA k-steps
  static constexpr int DS = SP + 8;                 // dense W row stride (bf16)
  static constexpr int KBYTES = RM * RS * (int)sizeof(T);
  static constexpr int DBYTES = 2 * RM * DS * 2;
  static constexpr int R1 = (KBYTES > DBYTES ? KBYTES : DBYTES);
  // k rows while the Gram entries are formed; then -W2 (hi | lo), later W1 (hi | lo)
  alignas(16) unsigned char r1[R1];
  alignas(16) T q[RM * RS];                         // q rows; bf16 input: then qe_hi
  alignas(16) uint16_t qhi[BF16IN ? 8 : RM * QS];
  alignas(16) uint16_t qlo[RM * QS];
  alignas(16) float lc[RM * kAR];                   // k.k Gram -> Lm rows
  alignas(16) float mc[RM * kAR];                   // q.k Gram -> Mm rows
  alignas(16) float wc[RM * kAR];                   // W1 rows (compact, by depth)
  alignas(16) int8_t anc[RM * kAR];                 // ancestor slot at each depth
  alignas(16) unsigned long long mask[RM];
  float alpha[RM], beta[RM], gamma[RM];
  int parent[RM];
  int8_t depth[RM];
  int bad;
  __device__ T *k() { return reinterpret_cast<T *>(r1); }
  __device__ uint16_t *dhi() { return reinterpret_cast<uint16_t *>(r1); }
  __device__ uint16_t *dlo() { return reinterpret_cast<uint16_t *>(r1) + RM * DS; }
};

__device__ __forceinline__ bf16x8 lds_frag(const uint16_t *row) {
  const uint4 u = *reinterpret_cast<const uint4 *>(row);
  return __builtin_bit_cast(bf16x8, u);
}

// x = hi + lo with hi, lo bf16 (round to nearest even); x - hi is exact in fp32.
__device__ __forceinline__ void split8(const float *x, bf16x8 &hi, bf16x8 &lo) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const __bf16 h = (__bf16)x[i];
    hi[i] = h;
    lo[i] = (__bf16)(x[i] - (float)h);
  }
}

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 8 consecutive elements from an LDS row (bf16 or fp32) widened to fp32.
__device__ __forceinline__ void lds_row8(const uint16_t *p, float *x) {
  const uint4 u = *reinterpret_cast<const uint4 *>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void lds_row8(const float *p, float *x) {
  const float4 a = *reinterpret_cast<const float4 *>(p);
  const float4 b = *reinterpret_cast<const float4 *>(p + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

// One 16x16 Gram tile (k-steps over d_k) from LDS rows ra (A) and rb (B).
template <int D, bool BF16IN>
__device__ __forceinline__ f32x4 gram_tile(const typename InT<BF16IN>::T *A,
                                           const typename InT<BF16IN>::T *Bm, int rs, int ra,
                                           int rb, int kofs) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    const int col = 32 * ks + kofs;
    if constexpr (BF16IN) {
      acc = mfma(lds_frag(A + ra * rs + col), lds_frag(Bm + rb * rs + col), acc);
    } else {
      float xa[8], xb[8];
      lds_row8(A + ra * rs + col, xa);
      lds_row8(Bm + rb * rs + col, xb);
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

// Load a padded compact row (20 floats) into registers.
__device__ __forceinline__ void load_row20(const float *p, float *r) {
#pragma unroll
  for (int v = 0; v < 5; ++v) {
    const float4 x = reinterpret_cast<const float4 *>(p)[v];
    r[4 * v] = x.x; r[4 * v + 1] = x.y; r[4 * v + 2] = x.z; r[4 * v + 3] = x.w;
  }
}
__device__ __forceinline__ void store_row20(float *p, const float *r) {
#pragma unroll
  for (int v = 0; v < 5; ++v)
    reinterpret_cast<float4 *>(p)[v] = make_float4(r[4 * v], r[4 * v + 1], r[4 * v + 2], r[4 * v + 3]);
}
__device__ __forceinline__ void load_anc20(const int8_t *p, int *a) {
  const uint4 u = *reinterpret_cast<const uint4 *>(p);
  const uint32_t t4 = *reinterpret_cast<const uint32_t *>(p + 16);
  const uint32_t w[5] = {u.x, u.y, u.z, u.w, t4};
#pragma unroll
  for (int e = 0; e < 20; ++e) a[e] = (int)((w[e >> 2] >> (8 * (e & 3))) & 0xffu);
}

// A transposed operand fragment: 8 consecutive node slots s (clamped to the used rows) of
// one channel column `col` of a row-major [node][H][D] input.
template <bool BF16IN, typename RowOff>
__device__ __forceinline__ void gather_t(const typename InT<BF16IN>::T *g, RowOff row_off, int n,
                                         int s0, int col, bf16x8 &hi, bf16x8 &lo) {
  if constexpr (BF16IN) {
    u16x8 f;
#pragma unroll
    for (int x = 0; x < 8; ++x) f[x] = g[row_off(min(s0 + x, n - 1)) + col];
    hi = __builtin_bit_cast(bf16x8, f);
  } else {
    float f[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) f[x] = g[row_off(min(s0 + x, n - 1)) + col];
    split8(f, hi, lo);
  }
}

template <int D, bool BF16IN, int NT, int W>
__global__ __launch_bounds__(64 * W, 2) void verify_kernel(VerifyParams p) {
  typedef VerifySmem<D, BF16IN, NT> SM;
  typedef typename SM::T T;
  constexpr int RS = SM::RS, QS = SM::QS, DS = SM::DS;
  constexpr int KS = D / 32;          // MFMA k-steps over d_k
  constexpr int KSS = SM::SP / 32;    // MFMA k-steps over the node axis
  constexpr int CH = 16 / sizeof(T);  // elements per 16-byte chunk
  constexpr int CPR = D / CH;         // 16-byte chunks per row
  constexpr int nthr = 64 * W;
  constexpr int S = D / (32 * W);     // d_v slices per head
  constexpr int NIS = D / 32;         // 32-channel slices of d_k
  __shared__ SM s;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g4 = lane >> 4, l16 = lane & 15;
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

  // ---- 0. loads ----------------------------------------------------------------------
  // Order matters: vector-memory loads complete in issue order, so the node metadata and
  // the k/q rows (needed first) are requested before the operand fragments of S0^T, V^T
  // and K^T, which then stream in while the tree prologue runs; the first barrier waits
  // only for the metadata and the k/q rows.
  if (tid == 0) s.bad = 0;
  for (int t = tid; t < n; t += nthr) {
    s.parent[t] = p.parent[(size_t)b * p.R + t];
    s.mask[t] = p.anc[(size_t)b * p.R + t];
    const size_t gi = (rowbase + t) * p.H + h;
    s.alpha[t] = load_elem(ga, gi);
    s.beta[t] = load_elem(gb, gi);
  }
  constexpr int KQPT = (2 * SM::RM * CPR + nthr - 1) / nthr;  // k/q chunks per thread
  constexpr int KQB = KQPT < 9 ? KQPT : 9;                     // staged in one batch
  const int nkq = 2 * n * CPR;
  auto kq_src = [&](int c) -> const T * {
    const int m = c / (n * CPR), rem = c - m * (n * CPR), t = rem / CPR, cc = rem - t * CPR;
    return (m ? gq : gk) + row_off(t) + cc * CH;
  };
  auto kq_dst = [&](int c) -> T * {
    const int m = c / (n * CPR), rem = c - m * (n * CPR), t = rem / CPR, cc = rem - t * CPR;
    return (m ? s.q : s.k()) + t * RS + cc * CH;
  };
  u32x4 kq[KQB];
#pragma unroll
  for (int i = 0; i < KQB; ++i) kq[i] = *reinterpret_cast<const u32x4 *>(kq_src(min(tid + i * nthr, nkq - 1)));

  const int j0 = js * 32 * W + wave * 32;
  const float *sbase = p.state + (size_t)hh * D * D;
  f32x4 sraw[2][KS][2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const f32x4 *ptr = reinterpret_cast<const f32x4 *>(sbase + (size_t)(j0 + 16 * mt + l16) * D + 32 * ks + 8 * g4);
      sraw[mt][ks][0] = ptr[0];
      sraw[mt][ks][1] = ptr[1];
    }
  // v: bf16 rows are parked in the (still unused) qe_lo region and gathered transposed
  // from there; fp32 rows are gathered transposed straight from memory
  constexpr int VPT = BF16IN ? (SM::RM * CPR + nthr - 1) / nthr : 1;
  u32x4 vpre[VPT];
  bf16x8 vt_hi[2][KSS], vt_lo[2][KSS];  // V^T rows j, node slots s
  if constexpr (BF16IN) {
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int c = min(tid + i * nthr, n * CPR - 1);
      vpre[i] = *reinterpret_cast<const u32x4 *>(gv + row_off(c / CPR) + (c % CPR) * CH);
    }
  } else {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int kk = 0; kk < KSS; ++kk)
        gather_t<BF16IN>(gv, row_off, n, 32 * kk + 8 * g4, j0 + 16 * mt + l16, vt_hi[mt][kk], vt_lo[mt][kk]);
  }
#pragma unroll
  for (int i = 0; i < KQB; ++i) {
    const int c = tid + i * nthr;
    if (c < nkq) *reinterpret_cast<u32x4 *>(kq_dst(c)) = kq[i];
  }
  for (int c = tid + KQB * nthr; c < nkq; c += nthr)  // only small workgroups get here
    *reinterpret_cast<u32x4 *>(kq_dst(c)) = *reinterpret_cast<const u32x4 *>(kq_src(c));
  __syncthreads();

  // ---- 1a. per node: validate links, ancestors from the bitmask, path gate ------------
  for (int t = tid; t < n; t += nthr) {
    const unsigned long long m = s.mask[t];
    const int dt = __popcll(m);
    const int pt = s.parent[t];
    const bool ok = (t == 0) ? (m == 0ull)
                             : (dt <= kMaxP && pt >= 0 && pt < t && m == (s.mask[pt] | (1ull << (t - 1))));
    if (!ok) s.bad = 1;
    // a[e] = slot of the ancestor at depth e (bit index + 1); 0 (the root) beyond the depth
    int a[kAR];
    unsigned long long mm = m;
    a[0] = 0;
#pragma unroll
    for (int e = 1; e < kAR; ++e) {
      a[e] = __ffsll((long long)mm);
      mm &= mm - 1;
    }
    uint32_t w[5];
#pragma unroll
    for (int v = 0; v < 5; ++v)
      w[v] = (uint32_t)a[4 * v] | ((uint32_t)a[4 * v + 1] << 8) | ((uint32_t)a[4 * v + 2] << 16) |
             ((uint32_t)a[4 * v + 3] << 24);
    *reinterpret_cast<uint4 *>(&s.anc[t * kAR]) = make_uint4(w[0], w[1], w[2], w[3]);
    *reinterpret_cast<uint32_t *>(&s.anc[t * kAR + 16]) = w[4];
    s.depth[t] = (int8_t)min(dt, kMaxP);
    float g = 1.f;
#pragma unroll
    for (int e = 0; e < kA; ++e) {
      const float ae = s.alpha[a[e]];
      g *= (e <= dt) ? ae : 1.f;
    }
    s.gamma[t] = g;
  }

  // K^T fragments of this wave's first d_k slice, from the k rows in LDS (bf16 input)
  bf16x8 kt_hi[2][KSS], kt_lo[2][KSS];
  if constexpr (BF16IN) {
#pragma unroll
    for (int it = 0; it < 2; ++it)
#pragma unroll
      for (int kk = 0; kk < KSS; ++kk) {
        u16x8 f;
#pragma unroll
        for (int x = 0; x < 8; ++x)
          f[x] = s.k()[min(32 * kk + 8 * g4 + x, n - 1) * RS + 32 * wave + 16 * it + l16];
        kt_hi[it][kk] = __builtin_bit_cast(bf16x8, f);
      }
  }

  // ---- 1b. Gram entries k_t.k_s and q_t.k_s for s ancestor-or-self of t (MFMA) --------
  {
    constexpr int NPAIR = NT * (NT + 1) / 2;
#pragma unroll
    for (int pi0 = 0; pi0 < 2 * NPAIR; pi0 += W) {
      const int pi = pi0 + wave;
      if (pi >= 2 * NPAIR) break;
      const int part = pi >= NPAIR;  // 0: k.k, 1: q.k
      const int qi = part ? pi - NPAIR : pi;
      int mt = 0;
      while ((mt + 1) * (mt + 2) / 2 <= qi) ++mt;
      const int nt = qi - mt * (mt + 1) / 2;
      if (16 * mt >= n) continue;
      const int ra = min(16 * mt + l16, n - 1), rb = min(16 * nt + l16, n - 1);
      const f32x4 g = gram_tile<D, BF16IN>(part ? s.q : s.k(), s.k(), RS, ra, rb, 8 * g4);
      const int sn = 16 * nt + l16;
      const unsigned long long ms = s.mask[rb];
      const int es = __popcll(ms);
      float *dst = part ? s.mc : s.lc;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * mt + 4 * g4 + r;
        const unsigned long long mtt = s.mask[min(t, n - 1)];
        const bool anc = sn == 0 || ((mtt >> (sn - 1)) & 1ull);
        if (t < n && sn <= t && es <= kMaxP && anc) dst[t * kAR + es] = g[r];
      }
    }
  }
  __syncthreads();
  if (s.bad) {
    const int jw0 = js * 32 * W, span = 32 * W;
    for (int c = tid; c < n * span; c += nthr) {
      const size_t oi = row_off(c / span) + jw0 + c % span;
      if (p.out_bf16) static_cast<uint16_t *>(p.o)[oi] = 0x7fc0;
      else static_cast<float *>(p.o)[oi] = __builtin_nanf("");
    }
    return;
  }

  // ---- 2. per node: Lm, Mm rows; then the Wm solve; W1 rows and the dense -W2 ---------
  if constexpr (BF16IN) {
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int c = tid + i * nthr;
      if (c < n * CPR) *reinterpret_cast<u32x4 *>(s.qlo + (c / CPR) * QS + (c % CPR) * CH) = vpre[i];
    }
  }
  for (int t = tid; t < n; t += nthr) {
    const int dt = s.depth[t];
    int arow[kAR];
    load_anc20(&s.anc[t * kAR], arow);
    float gk[kAR], gqk[kAR];
    load_row20(&s.lc[t * kAR], gk);
    load_row20(&s.mc[t * kAR], gqk);
    const float bt = s.beta[t];
    float rho = 1.f;  // g_t / g_{anc at depth e}
    float lrow[kAR], mrow[kAR];
#pragma unroll
    for (int e = kAR - 1; e >= 0; --e) {
      const bool on = e < kA && e <= dt;
      mrow[e] = on ? rho * gqk[e] : 0.f;
      lrow[e] = (e < dt) ? bt * rho * gk[e] : 0.f;
      const float ae = (e < kA) ? s.alpha[arow[e]] : 1.f;
      rho *= on ? ae : 1.f;
    }
    store_row20(&s.lc[t * kAR], lrow);
    store_row20(&s.mc[t * kAR], mrow);
  }
  __syncthreads();
  if constexpr (BF16IN) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int kk = 0; kk < KSS; ++kk) {
        u16x8 f;
#pragma unroll
        for (int x = 0; x < 8; ++x) f[x] = s.qlo[min(32 * kk + 8 * g4 + x, n - 1) * QS + j0 + 16 * mt + l16];
        vt_hi[mt][kk] = __builtin_bit_cast(bf16x8, f);
      }
  }
  for (int t = tid; t < n; t += nthr) {
    const int dt = s.depth[t];
    int arow[kAR];
    load_anc20(&s.anc[t * kAR], arow);
    float w[kAR];
    load_row20(&s.mc[t * kAR], w);  // Mm row, zero beyond the depth
    // right-looking solve of w (I + Lm) = Mm over the path, deepest ancestor first; for
    // depths beyond dt, w is zero and arow is the root, whose Lm row is zero
#pragma unroll
    for (int e2 = kA - 1; e2 >= 1; --e2) {
      float lr[kAR];
      load_row20(&s.lc[arow[e2] * kAR], lr);
#pragma unroll
      for (int e = 0; e < e2; ++e) w[e] -= w[e2] * lr[e];
    }
    float w1[kAR];
    uint16_t *dh = s.dhi() + t * DS, *dl = s.dlo() + t * DS;
#pragma unroll
    for (int v = 0; v < SM::SP / 8; ++v) {
      reinterpret_cast<u32x4 *>(dh)[v] = u32x4{0u, 0u, 0u, 0u};
      reinterpret_cast<u32x4 *>(dl)[v] = u32x4{0u, 0u, 0u, 0u};
    }
    // scatter -W2[t, anc at depth e] into column (slot) arow[e]; deepest first, so the
    // zero entries beyond the depth (all aimed at the root's column) land before e = 0
#pragma unroll
    for (int e = kAR - 1; e >= 0; --e) {
      const int sn = e < kA ? arow[e] : 0;
      const bool on = e < kA && e <= dt;
      w1[e] = on ? w[e] * s.beta[sn] : 0.f;
      const float m2 = -w1[e] * s.gamma[sn];
      const __bf16 hb = (__bf16)m2;
      dh[sn] = __builtin_bit_cast(uint16_t, hb);
      dl[sn] = __builtin_bit_cast(uint16_t, (__bf16)(m2 - (float)hb));
    }
    store_row20(&s.wc[t * kAR], w1);
  }
  __syncthreads();

  // ---- 3. effective queries: qe^T = g q^T - K^T W2^T (MFMA), split hi/lo (bf16) --------
  {
    uint16_t *qhi = BF16IN ? reinterpret_cast<uint16_t *>(s.q) : s.qhi;
    const int ntiles = (n + 15) / 16;
#pragma unroll
    for (int r = 0; r < (NIS + W - 1) / W; ++r) {
      const int is = wave + r * W;  // d_k slice of 32 channels
      if (is >= NIS) break;
      if (!BF16IN || r > 0) {
#pragma unroll
        for (int it = 0; it < 2; ++it)
#pragma unroll
          for (int kk = 0; kk < KSS; ++kk)
            gather_t<BF16IN>(gk, row_off, n, 32 * kk + 8 * g4, 32 * is + 16 * it + l16, kt_hi[it][kk], kt_lo[it][kk]);
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        if (nt >= ntiles) break;
        const int t = 16 * nt + l16, tb = min(t, n - 1);
        const float gt = s.gamma[tb];
        f32x4 acc[2];
#pragma unroll
        for (int it = 0; it < 2; ++it) {
          float x[4];
          const int i = 32 * is + 16 * it + 4 * g4;
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = gt * load_elem(s.q, (size_t)tb * RS + i + e);
          acc[it] = f32x4{x[0], x[1], x[2], x[3]};
        }
#pragma unroll
        for (int kk = 0; kk < KSS; ++kk) {
          const bf16x8 bh = lds_frag(s.dhi() + tb * DS + 32 * kk + 8 * g4);
          const bf16x8 bl = lds_frag(s.dlo() + tb * DS + 32 * kk + 8 * g4);
#pragma unroll
          for (int it = 0; it < 2; ++it) {
            acc[it] = mfma(kt_hi[it][kk], bh, acc[it]);
            acc[it] = mfma(kt_hi[it][kk], bl, acc[it]);
            if constexpr (!BF16IN) acc[it] = mfma(kt_lo[it][kk], bh, acc[it]);
          }
        }
        if (t < n) {
#pragma unroll
          for (int it = 0; it < 2; ++it) {
            const int i = 32 * is + 16 * it + 4 * g4;
            typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
            bf16x4 hv, lv;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              hv[e] = (__bf16)acc[it][e];
              lv[e] = (__bf16)(acc[it][e] - (float)hv[e]);
            }
            *reinterpret_cast<bf16x4 *>(qhi + t * QS + i) = hv;
            *reinterpret_cast<bf16x4 *>(s.qlo + t * QS + i) = lv;
          }
        }
      }
    }
  }
  __syncthreads();
  // the dense W1 (hi | lo) replaces -W2
  for (int t = tid; t < n; t += nthr) {
    int arow[kAR];
    load_anc20(&s.anc[t * kAR], arow);
    float w1[kAR];
    load_row20(&s.wc[t * kAR], w1);
    uint16_t *dh = s.dhi() + t * DS, *dl = s.dlo() + t * DS;
#pragma unroll
    for (int v = 0; v < SM::SP / 8; ++v) {
      reinterpret_cast<u32x4 *>(dh)[v] = u32x4{0u, 0u, 0u, 0u};
      reinterpret_cast<u32x4 *>(dl)[v] = u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int e = kAR - 1; e >= 0; --e) {
      const int sn = e < kA ? arow[e] : 0;
      const __bf16 hb = (__bf16)w1[e];
      dh[sn] = __builtin_bit_cast(uint16_t, hb);
      dl[sn] = __builtin_bit_cast(uint16_t, (__bf16)(w1[e] - (float)hb));
    }
  }
  __syncthreads();

  // ---- 4. o^T = S0^T [qe] + V^T W1^T (MFMA), node tile by node tile --------------------
  bf16x8 ahi[2][KS], alo[2][KS];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const float x[8] = {sraw[mt][ks][0][0], sraw[mt][ks][0][1], sraw[mt][ks][0][2], sraw[mt][ks][0][3],
                          sraw[mt][ks][1][0], sraw[mt][ks][1][1], sraw[mt][ks][1][2], sraw[mt][ks][1][3]};
      split8(x, ahi[mt][ks], alo[mt][ks]);
    }
  const uint16_t *qhi = BF16IN ? reinterpret_cast<const uint16_t *>(s.q) : s.qhi;
  const int ntiles = (n + 15) / 16;
  const int jl = j0 + 4 * g4;  // + 16*mt + r
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    if (nt >= ntiles) break;
    const int t = 16 * nt + l16;
    const int tb = min(t, n - 1);
    f32x4 acc0[2], acc1[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      acc0[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      acc1[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // S0^T qe: hi*hi into acc0, the cross terms into acc1
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int col = 32 * ks + 8 * g4;
      const bf16x8 bhi = lds_frag(qhi + tb * QS + col);
      const bf16x8 blo = lds_frag(s.qlo + tb * QS + col);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        acc0[mt] = mfma(ahi[mt][ks], bhi, acc0[mt]);
        acc1[mt] = mfma(alo[mt][ks], bhi, acc1[mt]);
        acc1[mt] = mfma(ahi[mt][ks], blo, acc1[mt]);
      }
    }
    // V^T W1^T over the node axis
#pragma unroll
    for (int kk = 0; kk < KSS; ++kk) {
      const bf16x8 wh = lds_frag(s.dhi() + tb * DS + 32 * kk + 8 * g4);
      const bf16x8 wl = lds_frag(s.dlo() + tb * DS + 32 * kk + 8 * g4);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        acc0[mt] = mfma(vt_hi[mt][kk], wh, acc0[mt]);
        acc1[mt] = mfma(vt_hi[mt][kk], wl, acc1[mt]);
        if constexpr (!BF16IN) acc1[mt] = mfma(vt_lo[mt][kk], wh, acc1[mt]);
      }
    }
    if (t < n) {
      const size_t ob = row_off(t);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const int j = jl + 16 * mt;
        const f32x4 o = acc0[mt] + acc1[mt];
        if (p.out_bf16) {
          typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
          const bf16x4 ob4 = {(__bf16)o[0], (__bf16)o[1], (__bf16)o[2], (__bf16)o[3]};
          *reinterpret_cast<bf16x4 *>(static_cast<uint16_t *>(p.o) + ob + j) = ob4;
        } else {
          *reinterpret_cast<f32x4 *>(static_cast<float *>(p.o) + ob + j) = o;
        }
      }
    }
  }
}

template <int D, bool BF16IN, int NT, int W>
hipError_t launch_w(const VerifyParams &p, hipStream_t stream) {
  const int HT = p.L * p.B * p.H;
  constexpr int S = D / (32 * W);
  const long long blocks = (S == 1) ? HT : (long long)((HT + 7) / 8) * 8 * S;
  hipLaunchKernelGGL((verify_kernel<D, BF16IN, NT, W>), dim3((unsigned)blocks), dim3(64 * W), 0,
                     stream, p);
  return hipGetLastError();
}

// Waves per workgroup (one per 32 value channels): a whole head per workgroup when there
// are enough heads to fill the chip, otherwise slices of a head across workgroups.
template <int D, bool BF16IN, int NT>
hipError_t launch_one(const VerifyParams &p, hipStream_t stream) {
  const int HT = p.L * p.B * p.H;
  if (HT >= 256) return launch_w<D, BF16IN, NT, D / 32>(p, stream);
  if (D == 128 && HT >= 128) return launch_w<D, BF16IN, NT, 2>(p, stream);
  return launch_w<D, BF16IN, NT, 1>(p, stream);
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
