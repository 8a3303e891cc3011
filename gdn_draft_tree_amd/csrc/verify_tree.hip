// Tree verify for Gated-DeltaNet layers on gfx950.
//
// What is computed (SpecPilot summary, Prerequisites > hybrid recurrent architecture):
// for every node t of a request's draft tree, with S_p the state of t's parent (the
// committed state S0 for the root),
//     S_t = a_t (I - b_t k_t k_t^T) S_p + b_t k_t v_t^T,      o_t = S_t^T q_t.
// The pages recompute states along root paths instead of snapshotting every node and name
// a WY-form kernel for it (Technical novelty).  This kernel never forms any node state.
//
// Tree form of the WY / UT transform.  Let g_t be the product of the gates a over the path
// root..t and, for an ancestor-or-self s of t, r(t,s) = g_t / g_s.  Writing
// S_t = g_t S0 + sum_{s on the path} r(t,s) k_s u_s^T, the pseudo-values u solve a system
// that is triangular along root paths, and the output collapses to
//     o_t = S0^T qe_t + sum_s W1[t,s] v_s,        qe_t = g_t q_t - sum_s W2[t,s] k_s,
// with W1 and W2 supported on the ancestors-or-self of t.  Scaling the unknowns by the
// path gates removes every gate from the system: if z solves, along t's path (depths
// e = 0..d_t, deepest first),
//     z[e] + sum_{e2 > e} z[e2] b_{anc e2} (k_{anc e2} . k_{anc e}) = q_t . k_{anc e},
// then W2[t, anc e] = g_t b_{anc e} z[e] and W1[t, anc e] = r(t, anc e) b_{anc e} z[e].
// So S0 (the only large operand, d_k x d_v fp32) is touched by ONE dense product
// [qe_t]^T S0 over all nodes, and everything that depends on the tree (Gram entries, the
// path solve) is O(nodes * depth) work.
//
// Work decomposition: one workgroup of four waves per (layer, request, head), two
// workgroups per CU (under 80 KiB of LDS and 256 registers per lane each), so that one
// head's HBM loads overlap the other head's arithmetic.  Per head:
//  0. the k and v rows go straight from HBM into LDS (buffer loads to LDS); tree masks and
//     gates into LDS; each wave loads the q operand fragments of its Gram tiles;
//  1. per node: ancestors from the bitmask, depth, path gate g_t; on MFMA, the Gram
//     entries k_t.k_s and q_t.k_s of ancestor pairs (16 x 16 tiles of the lower triangle),
//     kept compactly by the depth of s;
//  2. per node: the path solve for z (at most 16 steps), written as a dense fp32 row of
//     W1 in LDS;
//  3. per wave, its node tiles: qe^T = g q^T - K^T W2^T on MFMA, left in registers in
//     exactly the operand layout of the next product, then o^T = S0^T [qe] + V^T W1^T on
//     MFMA over the value channels, S0^T fragments loaded straight from HBM (the [d_v][d_k]
//     state layout makes them contiguous).  No barrier and no LDS write in this phase.
// S0, qe, W1 and W2 are split into hi + lo bf16 parts (hi*hi + lo*hi + hi*lo; the dropped
// lo*lo term is about 2^-16 relative); bf16 rows are used as given, fp32 rows are split too.

#include <type_traits>

#include "gdntree_internal.h"

namespace gdntree {
namespace {

constexpr int kA = kMaxAnc;  // 17 ancestor depths (0..16)
constexpr int kAR = 20;      // compact row padded to five 16-byte vectors

template <bool BF16IN>
struct InT;
template <>
struct InT<true> { typedef uint16_t T; };
template <>
struct InT<false> { typedef float T; };

template <int D, bool BF16IN, int NT>
struct VerifySmem {
  typedef typename InT<BF16IN>::T T;
  static constexpr int RM = (16 * NT < kMaxSlots) ? 16 * NT : kMaxSlots;  // node rows held
  static constexpr int CH = 16 / (int)sizeof(T);                          // elements per 16 B
  static constexpr int CPR = D / CH;                                      // chunks per row
  static constexpr int ROWB = (RM * D * (int)sizeof(T) + 1023) / 1024 * 1024;  // whole 1 KiB loads
  static constexpr int SP = (16 * NT + 31) / 32 * 32;  // node (contraction) axis of the products
  static constexpr int WS = SP + 4;                    // dense W1 row stride: conflict-free reads
  alignas(16) unsigned char krow[ROWB];
  alignas(16) unsigned char vrow[ROWB];
  alignas(16) float w1[RM * WS];
  alignas(16) float lc[RM * kAR];     // k_t . k_s, at the depth of s
  alignas(16) float mc[RM * kAR];     // q_t . k_s, at the depth of s
  alignas(16) int8_t anc[RM * kAR];   // slot of the ancestor at each depth (root beyond)
  alignas(16) unsigned long long mask[RM];
  alignas(16) float gamma[SP];        // path gate; zero past the node count
  float alpha[RM], beta[RM];
  int depth[RM];
  int bad;
};

// Rows live in LDS unpadded with their 16-byte chunks XOR-swizzled by the row index, so that
// 16 consecutive rows read at one logical column hit distinct banks.
template <int D, int CH>
__device__ __forceinline__ int swz(int r, int i) {
  constexpr int CPR = D / CH;
  return r * D + (((i / CH) ^ (r & (CPR - 1))) * CH) + (i % CH);
}

typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ bf16x8 frag16(const void *p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(p));
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

// Eight elements of one column of an LDS row block (rows r0..r0+7, clamped to rmax): the
// operand fragment of a product that contracts over the node axis.
template <int D, bool BF16IN>
__device__ __forceinline__ void col_frag(const typename InT<BF16IN>::T *rows, int r0, int rmax, int col,
                                        bf16x8 &hi, bf16x8 &lo) {
  constexpr int CH = 16 / (BF16IN ? 2 : 4);
  if constexpr (BF16IN) {
    u16x8 f;
#pragma unroll
    for (int x = 0; x < 8; ++x) f[x] = rows[swz<D, CH>(min(r0 + x, rmax), col)];
    hi = __builtin_bit_cast(bf16x8, f);
  } else {
    float f[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) f[x] = rows[swz<D, CH>(min(r0 + x, rmax), col)];
    split8(f, hi, lo);
  }
}

// Eight consecutive elements of one LDS row (a 16-byte chunk for bf16, two for fp32).
template <int D, bool BF16IN>
__device__ __forceinline__ void row_frag(const typename InT<BF16IN>::T *rows, int r, int col, bf16x8 &hi,
                                         bf16x8 &lo) {
  if constexpr (BF16IN) {
    hi = frag16(rows + swz<D, 8>(r, col));
  } else {
    const float4 a = *reinterpret_cast<const float4 *>(rows + swz<D, 4>(r, col));
    const float4 b = *reinterpret_cast<const float4 *>(rows + swz<D, 4>(r, col + 4));
    const float f[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    split8(f, hi, lo);
  }
}

// Gram work items: for part 0 (k rows) and 1 (q rows) and each 16-row tile mt, the tiles
// (mt, 0..mt) of [K; Q] K^T.  Items are dealt to the four waves largest first in a snake
// order, which balances the triangle (e.g. 8, 8, 7, 7 tiles at five node tiles).
__host__ __device__ constexpr int gram_item_wave(int k) { return ((k >> 2) & 1) ? 3 - (k & 3) : (k & 3); }
// register slot of the q operand of item k (odd k): q items of the same wave before it
__host__ __device__ constexpr int gram_qslot(int k) {
  int c = 0;
  for (int j = 1; j < k; j += 2) c += gram_item_wave(j) == gram_item_wave(k);
  return c;
}

template <int D, bool BF16IN, int NT>
__global__ __launch_bounds__(256, BF16IN ? 2 : 1) void verify_kernel(VerifyParams p) {
  typedef VerifySmem<D, BF16IN, NT> SM;
  typedef typename SM::T T;
  constexpr int RM = SM::RM, CH = SM::CH, CPR = SM::CPR, SP = SM::SP, WS = SM::WS;
  constexpr int KS = D / 32;               // MFMA k-steps over d_k
  constexpr int KSS = SP / 32;             // MFMA k-steps over the node axis
  constexpr int NTD = D / 16;              // 16-channel tiles of d_k (and of d_v)
  constexpr int QMAX = SM::ROWB / 1024;    // 1 KiB row-load instructions per matrix
  constexpr int QW = (QMAX + 3) / 4;       // ... per wave
  constexpr int NITEM = 2 * NT;
  constexpr int NQS = 2;                   // q-fragment slots per wave (max q items of a wave)
  constexpr int JPW = NTD / 4;             // value-channel tiles per wave
  constexpr int IPW = NTD / 4;             // effective-query d_k tiles per wave
  __shared__ SM s;

  const int tid = threadIdx.x, lane = tid & 63, g4 = lane >> 4, l16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = blockIdx.x;  // (layer, request, head)
  const int h = hh % p.H, lb = hh / p.H, b = lb % p.B;
  // n_nodes is read-only here: a scalar load
  const int32_t __attribute__((address_space(4))) *nn_c =
      (const int32_t __attribute__((address_space(4))) *)p.n_nodes;
  const int n = nn_c[b];
  if (n < 1 || n > p.R) return;  // no output for a request with an impossible node count
  const int nl = n - 1;
  const size_t rowbase = (size_t)lb * p.R;
  const size_t rstride = (size_t)p.H * D;  // elements between consecutive slots of one head
  const T *gq = static_cast<const T *>(p.q) + (rowbase * p.H + h) * (size_t)D;
  const T *gk = static_cast<const T *>(p.k) + (rowbase * p.H + h) * (size_t)D;
  const T *gv = static_cast<const T *>(p.v) + (rowbase * p.H + h) * (size_t)D;
  const T *krow = reinterpret_cast<const T *>(s.krow);
  const T *vrow = reinterpret_cast<const T *>(s.vrow);

  // ---- 0. loads ----------------------------------------------------------------------
  {
    // k and v rows -> LDS: each wave instruction fills 64 consecutive 16-byte chunks; lane l
    // of instruction q holds physical chunk 64 q + l and fetches the logical chunk that the
    // swizzle places there.  Chunks of rows past the node count fetch row n-1 (never used).
    const int nb = (int)(n * rstride * sizeof(T));
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void *)gk, 0, nb, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void *)gv, 0, nb, 0x00020000);
#pragma unroll
    for (int k = 0; k < QW; ++k) {
      const int qi = min(wave + 4 * k, QMAX - 1);
      const int pc = 64 * qi + lane, r = pc / CPR, c = (pc % CPR) ^ (r & (CPR - 1));
      const unsigned off = (unsigned)((min(r, nl) * (int)rstride + c * CH) * (int)sizeof(T));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void_t *)(s.krow + 1024 * qi), 16, off, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void_t *)(s.vrow + 1024 * qi), 16, off, 0, 0, 0);
    }
  }
  int par = 0;
  if (tid < n) {
    const size_t ti = (size_t)b * p.R + tid;
    par = p.parent[ti];
    s.mask[tid] = p.anc[ti];
    const size_t gi = (rowbase + tid) * p.H + h;
    s.alpha[tid] = load_elem(static_cast<const T *>(p.alpha), gi);
    s.beta[tid] = load_elem(static_cast<const T *>(p.beta), gi);
  }
  for (int i = tid; i < RM * kAR / 4; i += 256) {
    reinterpret_cast<float4 *>(s.lc)[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    reinterpret_cast<float4 *>(s.mc)[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  if (tid == 0) s.bad = 0;
  // q operand fragments (rows t = 16 mt + l16) of this wave's q Gram items
  bf16x8 qh[NQS][KS], ql[NQS][KS];
  {
#pragma unroll
    for (int k = 0; k < NITEM; ++k) {
      if ((k & 1) == 0 || gram_item_wave(k) != wave) continue;
      const int mt = NT - 1 - (k >> 1), slot = gram_qslot(k);
      if (16 * mt < n) {
        const T *qr = gq + (size_t)min(16 * mt + l16, nl) * rstride + 8 * g4;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          if constexpr (BF16IN) {
            qh[slot][ks] = frag16(qr + 32 * ks);
          } else {
            const float4 a = *reinterpret_cast<const float4 *>(qr + 32 * ks);
            const float4 c = *reinterpret_cast<const float4 *>(qr + 32 * ks + 4);
            const float f[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
            split8(f, qh[slot][ks], ql[slot][ks]);
          }
        }
      }
    }
  }
  __syncthreads();  // also waits for the row loads into LDS

  // ---- 1a. per node: validate links, ancestors from the bitmask, path gate --------------
  if (tid < n) {
    const int t = tid;
    const unsigned long long m = s.mask[t];
    const int dt = __popcll(m);
    const bool pin = par >= 0 && par < t;
    const bool ok = (t == 0) ? (m == 0ull)
                             : (dt <= kMaxP && pin && m == (s.mask[pin ? par : 0] | (1ull << (t - 1))));
    if (!ok) s.bad = 1;
    // a[e] = slot of the ancestor at depth e (bit index + 1); 0 (the root) beyond the depth
    // (clamped to the node count, which only an inconsistent mask can exceed)
    int a[kAR];
    unsigned long long mm = m;
    a[0] = 0;
#pragma unroll
    for (int e = 1; e < kAR; ++e) {
      a[e] = min(__ffsll((long long)mm), nl);
      mm &= mm - 1;
    }
    uint32_t w[5];
#pragma unroll
    for (int v = 0; v < 5; ++v)
      w[v] = (uint32_t)a[4 * v] | ((uint32_t)a[4 * v + 1] << 8) | ((uint32_t)a[4 * v + 2] << 16) |
             ((uint32_t)a[4 * v + 3] << 24);
    *reinterpret_cast<uint4 *>(&s.anc[t * kAR]) = make_uint4(w[0], w[1], w[2], w[3]);
    *reinterpret_cast<uint32_t *>(&s.anc[t * kAR + 16]) = w[4];
    s.depth[t] = min(dt, kMaxP);
    float g = 1.f;
#pragma unroll
    for (int e = 0; e < kA; ++e) {
      const float ae = s.alpha[a[e]];
      g *= (e <= dt) ? ae : 1.f;
    }
    s.gamma[t] = g;
  } else if (tid < SP) {
    s.gamma[tid] = 0.f;
  }

  // ---- 1b. Gram entries k_t.k_s and q_t.k_s for s ancestor-or-self of t (MFMA) ----------
  {
#pragma unroll
    for (int k = 0; k < NITEM; ++k) {
      if (gram_item_wave(k) != wave) continue;
      const int part = k & 1, mt = NT - 1 - (k >> 1), myslot = part ? gram_qslot(k) : 0;
      if (16 * mt >= n) continue;
      bf16x8 ah[KS], al[KS];
      if (part) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          ah[ks] = qh[myslot][ks];
          al[ks] = ql[myslot][ks];
        }
      } else {
        const int ra = min(16 * mt + l16, nl);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) row_frag<D, BF16IN>(krow, ra, 32 * ks + 8 * g4, ah[ks], al[ks]);
      }
      float *dst = part ? s.mc : s.lc;
      unsigned long long mrow[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) mrow[r] = s.mask[min(16 * mt + 4 * g4 + r, nl)];
#pragma unroll
      for (int nt = 0; nt <= mt; ++nt) {
        const int rb = min(16 * nt + l16, nl);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          bf16x8 bh, bl;
          row_frag<D, BF16IN>(krow, rb, 32 * ks + 8 * g4, bh, bl);
          acc = mfma(ah[ks], bh, acc);
          if constexpr (!BF16IN) {
            acc = mfma(al[ks], bh, acc);
            acc = mfma(ah[ks], bl, acc);
          }
        }
        const int sn = 16 * nt + l16;
        const int es = __popcll(s.mask[rb]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 16 * mt + 4 * g4 + r;
          const bool anc = sn == 0 || ((mrow[r] >> (sn - 1)) & 1ull);
          if (t < n && sn <= t && es <= kMaxP && anc) dst[t * kAR + es] = acc[r];
        }
      }
    }
  }
  __syncthreads();

  if (s.bad) {  // an inconsistent tree: NaN outputs for this request
    for (int c = tid; c < n * D; c += 256) {
      const size_t oi = ((rowbase + c / D) * p.H + h) * (size_t)D + c % D;
      if (p.out_bf16) static_cast<uint16_t *>(p.o)[oi] = 0x7fc0;
      else static_cast<float *>(p.o)[oi] = __builtin_nanf("");
    }
    return;
  }

  // this wave's value channels (tiles jt = JPW wave + q): their S0^T operand fragments are
  // loaded now and used last, so their HBM latency hides behind the path solve and the
  // effective queries.  The k
  // ordering inside a k-step matches the effective-query fragments (see phase 3):
  // elements 0..3 are d_k rows 32 ks + 4 g4 + 0..3, elements 4..7 rows 32 ks + 16 + 4 g4 + 0..3.
  f32x4 s0r[JPW][KS][2];
#pragma unroll
  for (int q = 0; q < JPW; ++q) {
    const float *sr = p.state + ((size_t)hh * D + 16 * (JPW * wave + q) + l16) * D + 4 * g4;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s0r[q][ks][0] = *reinterpret_cast<const f32x4 *>(sr + 32 * ks);
      s0r[q][ks][1] = *reinterpret_cast<const f32x4 *>(sr + 32 * ks + 16);
    }
  }
  // ---- 2. per node: the path solve, then the dense W1 row ---------------------------------
  if (tid < n) {
    const int t = tid, dt = s.depth[t];
    const uint4 ap = *reinterpret_cast<const uint4 *>(&s.anc[t * kAR]);
    const uint32_t ap4 = *reinterpret_cast<const uint32_t *>(&s.anc[t * kAR + 16]);
    auto anc_at = [&](int e) -> int {
      const uint32_t wd = e < 4 ? ap.x : e < 8 ? ap.y : e < 12 ? ap.z : e < 16 ? ap.w : ap4;
      return (int)((wd >> (8 * (e & 3))) & 0xffu);
    };
    float z[kAR];  // right-hand side q_t . k_{anc e}; zero beyond the depth
#pragma unroll
    for (int v = 0; v < 5; ++v) {
      const float4 x = reinterpret_cast<const float4 *>(&s.mc[t * kAR])[v];
      z[4 * v] = x.x; z[4 * v + 1] = x.y; z[4 * v + 2] = x.z; z[4 * v + 3] = x.w;
    }
    // deepest ancestor first; beyond the depth z is zero and the ancestor slot is the root
    // (a zero update).  Steps that no lane of the wave needs are skipped.
#pragma unroll
    for (int e2 = kMaxP; e2 >= 1; --e2) {
      if (__ballot(e2 <= dt) == 0) continue;
      const int a2 = anc_at(e2);
      const float c = z[e2] * s.beta[a2];
      const float4 *row = reinterpret_cast<const float4 *>(&s.lc[a2 * kAR]);
#pragma unroll
      for (int v = 0; v < (e2 + 3) / 4; ++v) {
        const float4 x = row[v];
        const float xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (4 * v + i < e2) z[4 * v + i] -= c * xs[i];
      }
    }
    float *wr = s.w1 + t * WS;
#pragma unroll
    for (int v = 0; v < SP / 4; ++v) reinterpret_cast<float4 *>(wr)[v] = make_float4(0.f, 0.f, 0.f, 0.f);
    // W1[t, anc e] = r(t, anc e) b_{anc e} z[e], with r(t, anc e) the gate product below e
    float rr = 1.f;
#pragma unroll
    for (int e = kA - 1; e >= 0; --e) {
      if (e <= dt) {
        const int ae = anc_at(e);
        wr[ae] = rr * s.beta[ae] * z[e];
        rr *= s.alpha[ae];
      }
    }
  }
  __syncthreads();

  // ---- 3. effective queries, then the outputs ---------------------------------------------
  // 3a. Each wave gathers its operand fragments that contract over the node axis from the k
  // and v rows: K^T for its d_k tiles (effective queries), V^T for its value channels.
  // q_t at rows i = 16 it + 4 g4 + 0..3 of this wave's effective-query tiles (used in 3b)
  typedef typename std::conditional<BF16IN, uint2, float4>::type QV;  // four q elements
  QV qv[NT][IPW];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const T *qr = gq + (size_t)min(16 * nt + l16, nl) * rstride + 16 * IPW * wave + 4 * g4;
#pragma unroll
    for (int q = 0; q < IPW; ++q) qv[nt][q] = *reinterpret_cast<const QV *>(qr + 16 * q);
  }

  const int ntl = (n + 15) / 16;  // node tiles in use
  bf16x8 kth[IPW][KSS], ktl[IPW][KSS], vth[JPW][KSS], vtl[JPW][KSS];
#pragma unroll
  for (int kk = 0; kk < KSS; ++kk) {
#pragma unroll
    for (int q = 0; q < IPW; ++q)
      col_frag<D, BF16IN>(krow, 32 * kk + 8 * g4, nl, 16 * (IPW * wave + q) + l16, kth[q][kk], ktl[q][kk]);
#pragma unroll
    for (int q = 0; q < JPW; ++q)
      col_frag<D, BF16IN>(vrow, 32 * kk + 8 * g4, nl, 16 * (JPW * wave + q) + l16, vth[q][kk], vtl[q][kk]);
  }
  __syncthreads();  // the k and v rows are dead: qe_hi and qe_lo (bf16) take their place

  // 3b. qe^T tiles C[i][t] = g_t q_t[i] - sum_s K^T[i][s] W2^T[s][t] for this wave's d_k tiles
  // and every node tile.  In the C layout a lane holds column t and rows 4 g4 + 0..3 of a
  // 16-row tile, so tiles 2 ks and 2 ks + 1 together are the k-step ks operand of lane
  // (g4, t) in the product with S0^T: one 16-byte chunk, stored at chunk 4 ks + g4 of row t
  // (XOR-swizzled by t so that the 16 rows read together hit distinct banks).
  uint16_t *qeh = reinterpret_cast<uint16_t *>(s.krow);
  uint16_t *qel = reinterpret_cast<uint16_t *>(s.vrow);
  constexpr int QCH = D / 8;  // 16-byte chunks per qe row
  auto qe_off = [&](int t, int chunk) { return t * D + ((chunk ^ (t & (QCH - 1))) * 8); };
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    if (nt >= ntl) break;
    const int t = 16 * nt + l16, tb = min(t, nl);
    bf16x8 w2h[KSS], w2l[KSS];  // -W1[t, s] g_s for s = 32 kk + 8 g4 + 0..7
#pragma unroll
    for (int kk = 0; kk < KSS; ++kk) {
      const float *wr = s.w1 + tb * WS + 32 * kk + 8 * g4;
      const float4 w0 = reinterpret_cast<const float4 *>(wr)[0], w1v = reinterpret_cast<const float4 *>(wr)[1];
      const float4 g0 = *reinterpret_cast<const float4 *>(&s.gamma[32 * kk + 8 * g4]);
      const float4 g1 = *reinterpret_cast<const float4 *>(&s.gamma[32 * kk + 8 * g4 + 4]);
      const float x[8] = {-w0.x * g0.x, -w0.y * g0.y, -w0.z * g0.z, -w0.w * g0.w,
                          -w1v.x * g1.x, -w1v.y * g1.y, -w1v.z * g1.z, -w1v.w * g1.w};
      split8(x, w2h[kk], w2l[kk]);
    }
    const float gt = s.gamma[tb];
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int q = 0; q < IPW; ++q) {
      f32x4 acc;
      if constexpr (BF16IN) {
        const uint2 u = qv[nt][q];
        acc[0] = gt * __uint_as_float(u.x << 16);
        acc[1] = gt * __uint_as_float(u.x & 0xffff0000u);
        acc[2] = gt * __uint_as_float(u.y << 16);
        acc[3] = gt * __uint_as_float(u.y & 0xffff0000u);
      } else {
        const float4 x = qv[nt][q];
        acc[0] = gt * x.x; acc[1] = gt * x.y; acc[2] = gt * x.z; acc[3] = gt * x.w;
      }
#pragma unroll
      for (int kk = 0; kk < KSS; ++kk) {
        acc = mfma(kth[q][kk], w2h[kk], acc);
        acc = mfma(kth[q][kk], w2l[kk], acc);
        if constexpr (!BF16IN) acc = mfma(ktl[q][kk], w2h[kk], acc);
      }
      bf16x4 hv, lv;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        hv[r] = (__bf16)acc[r];
        lv[r] = (__bf16)(acc[r] - (float)hv[r]);
      }
      if (t < n) {
        const int it = IPW * wave + q;  // d_k tile: k-step it / 2, half it % 2
        const int off = qe_off(t, 4 * (it >> 1) + g4) + 4 * (it & 1);
        *reinterpret_cast<bf16x4 *>(qeh + off) = hv;
        *reinterpret_cast<bf16x4 *>(qel + off) = lv;
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // one node tile's loads in flight at a time
  }
  __syncthreads();

  // 3c. o^T = S0^T [qe] + V^T W1^T for this wave's value channels, node tile by node tile
  bf16x8 ah[JPW][KS], al[JPW][KS];
#pragma unroll
  for (int q = 0; q < JPW; ++q)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      // split here, not earlier: the raw and the split fragments are never live together
      asm volatile("" : "+v"(s0r[q][ks][0]), "+v"(s0r[q][ks][1]));
      const float x[8] = {s0r[q][ks][0][0], s0r[q][ks][0][1], s0r[q][ks][0][2], s0r[q][ks][0][3],
                          s0r[q][ks][1][0], s0r[q][ks][1][1], s0r[q][ks][1][2], s0r[q][ks][1][3]};
      split8(x, ah[q][ks], al[q][ks]);
    }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    if (nt >= ntl) break;
    const int t = 16 * nt + l16, tb = min(t, nl);
    f32x4 acc0[JPW], acc1[JPW];
#pragma unroll
    for (int q = 0; q < JPW; ++q) {
      acc0[q] = f32x4{0.f, 0.f, 0.f, 0.f};
      acc1[q] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int off = qe_off(tb, 4 * ks + g4);
      const bf16x8 bh = frag16(qeh + off), bl = frag16(qel + off);
#pragma unroll
      for (int q = 0; q < JPW; ++q) {
        acc0[q] = mfma(ah[q][ks], bh, acc0[q]);
        acc1[q] = mfma(al[q][ks], bh, acc1[q]);
        acc1[q] = mfma(ah[q][ks], bl, acc1[q]);
      }
    }
#pragma unroll
    for (int kk = 0; kk < KSS; ++kk) {  // W1[t, s] for s = 32 kk + 8 g4 + 0..7
      const float *wr = s.w1 + tb * WS + 32 * kk + 8 * g4;
      const float4 w0 = reinterpret_cast<const float4 *>(wr)[0], w1v = reinterpret_cast<const float4 *>(wr)[1];
      const float x[8] = {w0.x, w0.y, w0.z, w0.w, w1v.x, w1v.y, w1v.z, w1v.w};
      bf16x8 wh, wl;
      split8(x, wh, wl);
#pragma unroll
      for (int q = 0; q < JPW; ++q) {
        acc0[q] = mfma(vth[q][kk], wh, acc0[q]);
        acc1[q] = mfma(vth[q][kk], wl, acc1[q]);
        if constexpr (!BF16IN) acc1[q] = mfma(vtl[q][kk], wh, acc1[q]);
      }
    }
    if (t < n) {
#pragma unroll
      for (int q = 0; q < JPW; ++q) {
        const f32x4 o = acc0[q] + acc1[q];
        const size_t ob = ((rowbase + t) * p.H + h) * (size_t)D + 16 * (JPW * wave + q) + 4 * g4;
        if (p.out_bf16) {
          typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
          const bf16x4 o4 = {(__bf16)o[0], (__bf16)o[1], (__bf16)o[2], (__bf16)o[3]};
          *reinterpret_cast<bf16x4 *>(static_cast<uint16_t *>(p.o) + ob) = o4;
        } else {
          *reinterpret_cast<f32x4 *>(static_cast<float *>(p.o) + ob) = o;
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int D, bool BF16IN, int NT>
hipError_t launch_one(const VerifyParams &p, hipStream_t stream) {
  const int units = p.L * p.B * p.H;
  hipLaunchKernelGGL((verify_kernel<D, BF16IN, NT>), dim3((unsigned)units), dim3(256), 0, stream, p);
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
