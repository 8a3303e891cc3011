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
// root..t.  Unrolling the recurrence along t's path gives S_t = g_t S0 + sum_s (g_t/g_s)
// k_s u_s^T over the ancestors-or-self s of t, where the pseudo-values u solve a system that
// is triangular along root paths with right-hand side b_s v'_s,
//     v'_s = v_s - g_s S0^T k_s,
// and the readout collapses to
//     o_t = g_t S0^T q_t + sum_s W1[t,s] v'_s.
// W1 is supported on the ancestors-or-self of t.  Scaling the unknowns by the path gates
// removes every gate from the system: if z solves, along t's path (depths e = 0..d_t,
// deepest first),
//     z[e] + sum_{e2 > e} z[e2] b_{anc e2} (k_{anc e2} . k_{anc e}) = q_t . k_{anc e},
// then W1[t, anc e] = (g_t / g_{anc e}) b_{anc e} z[e].
// So S0, the only large operand (d_k x d_v fp32), enters through ONE dense product
// [Q; K] S0 that does not depend on the tree at all, and the tree enters through small
// O(nodes * depth) work (Gram entries of ancestor pairs, the path solve) and one dense
// node x node product W1 V'.
//
// Work decomposition: one workgroup of four waves per (layer, request, head), two
// workgroups per CU.  Wave w owns value channels [32 w, 32 w + 32) (d = 128).  Per head:
//  0. q, k, v rows go straight from HBM into LDS (buffer loads to LDS); tree masks and
//     gates into LDS; each wave loads its S0 operand fragments into registers;
//  1. every wave: P_Q = Q S0 and P_K = K S0 for its channels on MFMA (S0 split hi + lo
//     bf16, rows exact in bf16), the C tiles kept in registers.  Waves 1-3 also compute the
//     Gram tiles [Q; K] K^T of the lower node triangle on MFMA and keep the entries of
//     ancestor pairs, compactly by the depth of the ancestor.  Wave 0 reads each node's
//     ancestors from its bitmask and forms the path gate g_t;
//  2. wave 0: one lane per node solves its path system and writes the node's W1 row (hi +
//     lo bf16) to LDS; every wave: V' = V - g P_K for its channels (V enters the C tiles
//     through a product with a 0/1 selector, so no transposed read of V is needed);
//  3. every wave: o = g P_Q + W1 V' on MFMA (the C layout of V' is exactly the B-operand
//     layout the product needs), then the stores.
// Three barriers per head.

#include <type_traits>

#include "gdntree_internal.h"

namespace gdntree {
namespace {

constexpr int kAR = 20;  // compact row: ancestor depths 0..16, padded to five 16-byte vectors

template <bool BF16IN>
struct InT;
template <>
struct InT<true> { typedef uint16_t T; };
template <>
struct InT<false> { typedef float T; };

template <int D, bool BF16IN, int NT>
struct VerifySmem {
  typedef typename InT<BF16IN>::T T;
  static constexpr int RM = (16 * NT < kMaxSlots) ? 16 * NT : kMaxSlots;   // node rows held
  static constexpr int ROWB = (RM * D * (int)sizeof(T) + 1023) / 1024 * 1024;  // whole 1 KiB loads
  static constexpr int SP = (16 * NT + 31) / 32 * 32;  // node (contraction) axis of W1 V'
  static constexpr int W1B = 2 * RM * SP * 2;          // W1 rows, hi and lo bf16
  static constexpr int QKB = (2 * ROWB > W1B) ? 2 * ROWB : W1B;
  alignas(16) unsigned char qk[QKB];   // q rows, k rows; W1 after phase 1
  alignas(16) unsigned char vrow[ROWB];
  alignas(16) float lc[RM * kAR];      // k_t . k_s for s a strict ancestor of t, at depth(s)
  alignas(16) float mc[RM * kAR];      // q_t . k_s for s an ancestor-or-self of t, at depth(s)
  alignas(16) unsigned long long mask[RM];
  alignas(16) float gamma[16 * NT];    // path gate; zero past the node count
  float alpha[RM], beta[RM];
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

// Eight consecutive elements of one LDS row (a 16-byte chunk for bf16, two for fp32): the
// operand fragment of a product that contracts over d.
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

// Position of node s inside its 32-node chunk of a W1 row.  The B operand of W1 V' is V' in
// the C layout of two 16-node tiles: lane (g, c) holds nodes 4 g + 0..3 of the first tile and
// 16 + 4 g + 0..3 of the second, so the k index 8 g + e of the product stands for node
// 4 g + e (e < 4) or 16 + 4 g + e - 4 (e >= 4); W1 rows are stored in that k order.
__device__ __forceinline__ int w1_pos(int s) {
  const int sl = s & 31;
  return (s & ~31) + 8 * ((sl & 15) >> 2) + ((sl >> 4) << 2) + (sl & 3);
}

__device__ __forceinline__ int wave_max_i32(int x) {
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x121, 0xf, 0xf, false));  // row_ror 1
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x122, 0xf, 0xf, false));  // row_ror 2
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x124, 0xf, 0xf, false));  // row_ror 4
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x128, 0xf, 0xf, false));  // row_ror 8
  const int r0 = __builtin_amdgcn_readlane(x, 0), r1 = __builtin_amdgcn_readlane(x, 16);
  const int r2 = __builtin_amdgcn_readlane(x, 32), r3 = __builtin_amdgcn_readlane(x, 48);
  return max(max(r0, r1), max(r2, r3));
}

// Barrier that orders LDS only: every wave's LDS traffic is complete, in-flight HBM loads
// into registers are not waited for.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
}

template <int D, bool BF16IN, int NT>
__global__ __launch_bounds__(256, BF16IN ? 2 : 1) void verify_kernel(VerifyParams p) {
  typedef VerifySmem<D, BF16IN, NT> SM;
  typedef typename SM::T T;
  constexpr int RM = SM::RM, SP = SM::SP;
  constexpr int CH = 16 / (int)sizeof(T), CPR = D / CH;
  constexpr int KS = D / 32;               // MFMA k-steps over d_k
  constexpr int KSS = SP / 32;             // MFMA k-steps over the node axis
  constexpr int JPW = D / 64;              // 16-channel value tiles per wave
  constexpr int QMAX = SM::ROWB / 1024;    // 1 KiB row-load instructions per matrix
  constexpr int NS0 = JPW * KS * 2;        // S0 fragment loads per lane
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
  const int ntl = (n + 15) / 16;  // node tiles in use
  const size_t rowbase = (size_t)lb * p.R;
  const size_t rstride = (size_t)p.H * D;  // elements between consecutive slots of one head
  const T *gq = static_cast<const T *>(p.q) + (rowbase * p.H + h) * (size_t)D;
  const T *gk = static_cast<const T *>(p.k) + (rowbase * p.H + h) * (size_t)D;
  const T *gv = static_cast<const T *>(p.v) + (rowbase * p.H + h) * (size_t)D;
  const T *qrow = reinterpret_cast<const T *>(s.qk);
  const T *krow = reinterpret_cast<const T *>(s.qk + SM::ROWB);
  const T *vrow = reinterpret_cast<const T *>(s.vrow);
  uint16_t *w1h = reinterpret_cast<uint16_t *>(s.qk);
  uint16_t *w1l = w1h + RM * SP;

  // ---- 0. loads ----------------------------------------------------------------------
  // tree masks, gates and parents: raw loads, converted only after every HBM load is issued
  // (unconditional loads at a clamped slot, so that no branch forces an early wait)
  const int tcl = min(tid, nl);
  const unsigned long long my_mask = p.anc[(size_t)b * p.R + tcl];
  const T my_alpha = static_cast<const T *>(p.alpha)[(rowbase + tcl) * p.H + h];
  const T my_beta = static_cast<const T *>(p.beta)[(rowbase + tcl) * p.H + h];
  int my_par = -1;
  if (wave == 0 && lane + 1 < n) my_par = p.parent[(size_t)b * p.R + lane + 1];
  __builtin_amdgcn_sched_barrier(0);
  {
    // q, k, v rows -> LDS: each wave instruction fills 64 consecutive 16-byte chunks; lane l
    // of instruction qi holds physical chunk 64 qi + l and fetches the logical chunk that the
    // swizzle places there.  Chunks of rows past the node count fetch row n-1 (never used).
    const int nb = (int)(n * rstride * sizeof(T));
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc((void *)gq, 0, nb, 0x00020000);
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void *)gk, 0, nb, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void *)gv, 0, nb, 0x00020000);
#pragma unroll
    for (int x = 0; x < (3 * QMAX + 3) / 4; ++x) {
      const int item = wave + 4 * x;
      if (item >= 3 * QMAX) break;
      const int mat = item / QMAX, qi = item % QMAX;
      const int pc = 64 * qi + lane, r = pc / CPR, c = (pc % CPR) ^ (r & (CPR - 1));
      const unsigned off = (unsigned)((min(r, nl) * (int)rstride + c * CH) * (int)sizeof(T));
      unsigned char *dst = (mat == 2 ? s.vrow : s.qk + mat * SM::ROWB) + 1024 * qi;
      const __amdgpu_buffer_rsrc_t rs = mat == 0 ? rq : (mat == 1 ? rk : rv);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t *)dst, 16, off, 0, 0, 0);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  // S0 operand fragments of this wave's value channels (B operand of X S0: lane (g, c) holds
  // S0[32 ks + 8 g + 0..7][channel c], contiguous in the [d_v][d_k] state layout).
  f32x4 s0r[JPW][KS][2];
#pragma unroll
  for (int j = 0; j < JPW; ++j) {
    const float *sr = p.state + ((size_t)hh * D + 16 * (JPW * wave + j) + l16) * D + 8 * g4;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s0r[j][ks][0] = *reinterpret_cast<const f32x4 *>(sr + 32 * ks);
      s0r[j][ks][1] = *reinterpret_cast<const f32x4 *>(sr + 32 * ks + 4);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  if (tid < n) {
    s.mask[tid] = my_mask;
    s.alpha[tid] = load_elem(&my_alpha, 0);
    s.beta[tid] = load_elem(&my_beta, 0);
  } else if (tid < 16 * NT) {
    s.gamma[tid] = 0.f;
  }
  for (int i = tid; i < RM * kAR / 4; i += 256) {
    reinterpret_cast<float4 *>(s.lc)[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    reinterpret_cast<float4 *>(s.mc)[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  if (tid == 0) s.bad = 0;
  // the row loads (issued before the S0 loads) have landed; S0 may still be in flight
  __builtin_amdgcn_s_waitcnt(0x0070 | ((NS0 & 15) | ((NS0 >> 4) << 14)));  // vmcnt(NS0) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();

  // ---- 1a. wave 0: per node, ancestors from the bitmask, depth, path gate ---------------
  // Lane l of wave 0 owns node l + 1 (through phase 2); the root is handled by wave 1.
  const int t_me = lane + 1;
  uint32_t ancw[5] = {0u, 0u, 0u, 0u, 0u};  // slot of the ancestor at depth e, byte e
  int d_me = 0;
  if (wave == 0 && t_me < n) {
    const unsigned long long m = s.mask[t_me];
    d_me = __popcll(m);
    const bool pin = my_par >= 0 && my_par < t_me;
    const bool ok = d_me <= kMaxP && pin && m == (s.mask[pin ? my_par : 0] | (1ull << (t_me - 1)));
    if (!ok) s.bad = 1;
    d_me = min(d_me, kMaxP);
    unsigned long long mm = m;
    float g = s.alpha[0];
#pragma unroll
    for (int e = 1; e <= kMaxP; ++e) {
      const int a = min(__ffsll((long long)mm), nl);  // 0 (the root) beyond the depth
      mm &= mm - 1;
      ancw[e >> 2] |= (uint32_t)a << (8 * (e & 3));
      const float ae = s.alpha[a];
      g *= (e <= d_me) ? ae : 1.f;
    }
    s.gamma[t_me] = g;
  } else if (wave == 1 && lane == 0) {
    s.gamma[0] = s.alpha[0];
    if (s.mask[0] != 0ull) s.bad = 1;
  }

  // ---- 1b. P_Q = Q S0, P_K = K S0 (all waves); Gram tiles (waves 1-3) ---------------------
  bf16x8 s0h[JPW][KS], s0l[JPW][KS];
#pragma unroll
  for (int j = 0; j < JPW; ++j)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const float x[8] = {s0r[j][ks][0][0], s0r[j][ks][0][1], s0r[j][ks][0][2], s0r[j][ks][0][3],
                          s0r[j][ks][1][0], s0r[j][ks][1][1], s0r[j][ks][1][2], s0r[j][ks][1][3]};
      split8(x, s0h[j][ks], s0l[j][ks]);
    }
  // P_Q is kept transposed (lane (g, t) holds P_Q[t][4 g + 0..3] of a channel tile: the C
  // layout of S0^T Q^T), P_K in the node-major C layout (lane (g, c) holds P_K[4 g + 0..3][c]).
  // Both come from the same registers: S0 fragments serve as the A operand of one product
  // and the B operand of the other, and so do the row fragments.
  f32x4 pqt[NT][JPW], pk[NT][JPW];
#pragma unroll
  for (int mt = 0; mt < NT; ++mt) {
#pragma unroll
    for (int j = 0; j < JPW; ++j) {
      pqt[mt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
      pk[mt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if (mt >= ntl) continue;
    const int tme = 16 * mt + l16, ra = min(tme, nl);
    bf16x8 aqh[KS], aql[KS], akh[KS], akl[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      row_frag<D, BF16IN>(qrow, ra, 32 * ks + 8 * g4, aqh[ks], aql[ks]);
      row_frag<D, BF16IN>(krow, ra, 32 * ks + 8 * g4, akh[ks], akl[ks]);
    }
#pragma unroll
    for (int j = 0; j < JPW; ++j)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        pqt[mt][j] = mfma(s0h[j][ks], aqh[ks], pqt[mt][j]);
        pqt[mt][j] = mfma(s0l[j][ks], aqh[ks], pqt[mt][j]);
        pk[mt][j] = mfma(akh[ks], s0h[j][ks], pk[mt][j]);
        pk[mt][j] = mfma(akh[ks], s0l[j][ks], pk[mt][j]);
        if constexpr (!BF16IN) {
          pqt[mt][j] = mfma(s0h[j][ks], aql[ks], pqt[mt][j]);
          pk[mt][j] = mfma(akl[ks], s0h[j][ks], pk[mt][j]);
        }
      }
    // Gram tiles, transposed: tile (nt <= mt) holds k_s . k_t and k_s . q_t with lane (g, t)
    // owning node t = 16 mt + l16 and s = 16 nt + 4 g + 0..3.  Tile pair i = mt (mt + 1) / 2
    // + nt goes to wave 1 + i % 3.
    if (wave == 0) continue;
    const unsigned long long tmask = s.mask[ra];
    const int trow = ra * kAR;
#pragma unroll
    for (int nt = 0; nt <= mt; ++nt) {
      if (1 + (mt * (mt + 1) / 2 + nt) % 3 != wave) continue;
      const int rb = min(16 * nt + l16, nl);
      f32x4 gk4 = {0.f, 0.f, 0.f, 0.f}, gq4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        bf16x8 bh, bl;
        row_frag<D, BF16IN>(krow, rb, 32 * ks + 8 * g4, bh, bl);
        gk4 = mfma(bh, akh[ks], gk4);
        gq4 = mfma(bh, aqh[ks], gq4);
        if constexpr (!BF16IN) {
          gk4 = mfma(bl, akh[ks], gk4);
          gk4 = mfma(bh, akl[ks], gk4);
          gq4 = mfma(bl, aqh[ks], gq4);
          gq4 = mfma(bh, aql[ks], gq4);
        }
      }
      // keep the entries of ancestor pairs at depth(s) = the number of t's ancestors in slots
      // 1..s; everything else goes to the unused padding entries 17..19 of t's row (no branch)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int sn = 16 * nt + 4 * g4 + i;
        const unsigned long long below = sn >= 64 ? ~0ull : ((1ull << sn) - 1ull);
        const int es = __popcll(tmask & below);
        const bool anc = sn == 0 || ((tmask >> ((sn - 1) & 63)) & 1ull);
        const bool keep = tme < n && sn <= tme && anc && es <= kMaxP;
        const int dummy = trow + kMaxAnc + (i % 3);
        s.mc[keep ? trow + es : dummy] = gq4[i];
        s.lc[keep && sn != tme ? trow + es : dummy] = gk4[i];
      }
    }
  }
  lds_barrier();

  if (s.bad) {  // an inconsistent tree: NaN outputs for this request
    for (int c = tid; c < n * D; c += 256) {
      const size_t oi = ((rowbase + c / D) * p.H + h) * (size_t)D + c % D;
      if (p.out_bf16) static_cast<uint16_t *>(p.o)[oi] = 0x7fc0;
      else static_cast<float *>(p.o)[oi] = __builtin_nanf("");
    }
    return;
  }

  // ---- 2a. V' = V - g P_K for this wave's channels, packed as the B operand of W1 V' ------
  // V enters the C tiles through one product with a 0/1 selector B[k][c] = (k == c + off):
  // the A operand is a plain row fragment of V, so V is never read transposed.
  bf16x8 vph[KSS][JPW], vpl[KSS][JPW];
  {
    bf16x8 isel[JPW];
#pragma unroll
    for (int j = 0; j < JPW; ++j) {
      const int off = 16 * ((JPW * wave + j) & 1);
#pragma unroll
      for (int e = 0; e < 8; ++e) isel[j][e] = (__bf16)((8 * g4 + e == l16 + off) ? 1.f : 0.f);
    }
    const int vcol = 32 * ((JPW * wave) >> 1) + 8 * g4;  // this wave's 32-channel chunk
#pragma unroll
    for (int mt = 0; mt < 2 * KSS; ++mt) {
      f32x4 vp[JPW];
#pragma unroll
      for (int j = 0; j < JPW; ++j) vp[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (mt < NT && mt < ntl) {
        const int mc_ = mt < NT ? mt : NT - 1;  // (static index; mt < NT here)
        const float4 gm = *reinterpret_cast<const float4 *>(&s.gamma[16 * mt + 4 * g4]);
        bf16x8 avh, avl;
        row_frag<D, BF16IN>(vrow, min(16 * mt + l16, nl), vcol, avh, avl);
#pragma unroll
        for (int j = 0; j < JPW; ++j) {
          vp[j][0] = -gm.x * pk[mc_][j][0];
          vp[j][1] = -gm.y * pk[mc_][j][1];
          vp[j][2] = -gm.z * pk[mc_][j][2];
          vp[j][3] = -gm.w * pk[mc_][j][3];
          vp[j] = mfma(avh, isel[j], vp[j]);
          if constexpr (!BF16IN) vp[j] = mfma(avl, isel[j], vp[j]);
        }
      }
#pragma unroll
      for (int j = 0; j < JPW; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const __bf16 hv = (__bf16)vp[j][i];
          vph[mt >> 1][j][4 * (mt & 1) + i] = hv;
          vpl[mt >> 1][j][4 * (mt & 1) + i] = (__bf16)(vp[j][i] - (float)hv);
        }
    }
  }

  // ---- 2b. path solve, one lane of wave 0 per node; the root by wave 1 ------------------
  if (wave == 0) {
    const int dmax = wave_max_i32(t_me < n ? d_me : 0);
    if (t_me < n) {
      const int t = t_me;
      auto anc_at = [&](int e) -> int { return (int)((ancw[e >> 2] >> (8 * (e & 3))) & 0xffu); };
      float z[kAR];  // right-hand side q_t . k_{anc e}; zero beyond the depth
#pragma unroll
      for (int v = 0; v < kAR / 4; ++v) {
        const float4 x = reinterpret_cast<const float4 *>(&s.mc[t * kAR])[v];
        z[4 * v] = x.x; z[4 * v + 1] = x.y; z[4 * v + 2] = x.z; z[4 * v + 3] = x.w;
      }
      float bet[kMaxAnc];
#pragma unroll
      for (int e = 0; e <= kMaxP; ++e) bet[e] = s.beta[anc_at(e)];
      // deepest ancestor first; beyond a lane's depth z is zero and the ancestor slot is the
      // root, so those steps change nothing.  Steps deeper than every lane are skipped.
#pragma unroll
      for (int e2 = kMaxP; e2 >= 1; --e2) {
        if (e2 > dmax) continue;
        const float c = z[e2] * bet[e2];
        const float4 *row = reinterpret_cast<const float4 *>(&s.lc[anc_at(e2) * kAR]);
#pragma unroll
        for (int v = 0; v < (e2 + 3) / 4; ++v) {
          const float4 x = row[v];
          const float xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (4 * v + i < e2) z[4 * v + i] -= c * xs[i];
        }
      }
      // W1[t, anc e] = (g_t / g_{anc e}) b_{anc e} z[e]; the gate ratio is the product of the
      // gates strictly below depth e on the path
      uint4 *rh = reinterpret_cast<uint4 *>(w1h + t * SP);
      uint4 *rl = reinterpret_cast<uint4 *>(w1l + t * SP);
#pragma unroll
      for (int v = 0; v < SP / 8; ++v) {
        rh[v] = make_uint4(0u, 0u, 0u, 0u);
        rl[v] = make_uint4(0u, 0u, 0u, 0u);
      }
      float rr = 1.f;
#pragma unroll
      for (int e = kMaxP; e >= 0; --e) {
        if (e <= d_me) {
          const int ae = anc_at(e);
          const float w = rr * bet[e] * z[e];
          const __bf16 hv = (__bf16)w;
          const __bf16 lv = (__bf16)(w - (float)hv);
          const int pos = t * SP + w1_pos(ae);
          w1h[pos] = __builtin_bit_cast(uint16_t, hv);
          w1l[pos] = __builtin_bit_cast(uint16_t, lv);
          rr *= s.alpha[ae];
        }
      }
    }
  } else if (wave == 1 && lane == 0) {
    // the root: W1[0, 0] = b_0 (q_0 . k_0)
    uint4 *rh = reinterpret_cast<uint4 *>(w1h);
    uint4 *rl = reinterpret_cast<uint4 *>(w1l);
#pragma unroll
    for (int v = 0; v < SP / 8; ++v) {
      rh[v] = make_uint4(0u, 0u, 0u, 0u);
      rl[v] = make_uint4(0u, 0u, 0u, 0u);
    }
    const float w = s.beta[0] * s.mc[0];
    const __bf16 hv = (__bf16)w;
    w1h[0] = __builtin_bit_cast(uint16_t, hv);
    w1l[0] = __builtin_bit_cast(uint16_t, (__bf16)(w - (float)hv));
  }
  lds_barrier();

  // ---- 3. o^T = g P_Q^T + V'^T W1^T for this wave's value channels, node tile by node tile --
  // A operand: V' (its registers are exactly the A layout of V'^T), B operand: W1 rows from
  // LDS.  Lane (g, t) ends with o[t][16 jt + 4 g + 0..3]: one 8-byte (bf16) store per tile.
  const size_t ostride = (size_t)p.H * D;
  const size_t obase = (rowbase * p.H + h) * (size_t)D;
#pragma unroll
  for (int mt = 0; mt < NT; ++mt) {
    if (mt >= ntl) break;
    const int t = 16 * mt + l16, tr = min(t, nl);
    const float gt = s.gamma[t];
    f32x4 acc[JPW];
#pragma unroll
    for (int j = 0; j < JPW; ++j) acc[j] = gt * pqt[mt][j];
#pragma unroll
    for (int kk = 0; kk < KSS; ++kk) {
      const bf16x8 wh = frag16(w1h + tr * SP + 32 * kk + 8 * g4);
      const bf16x8 wl = frag16(w1l + tr * SP + 32 * kk + 8 * g4);
#pragma unroll
      for (int j = 0; j < JPW; ++j) {
        acc[j] = mfma(vph[kk][j], wh, acc[j]);
        acc[j] = mfma(vpl[kk][j], wh, acc[j]);
        acc[j] = mfma(vph[kk][j], wl, acc[j]);
      }
    }
    if (t < n) {
#pragma unroll
      for (int j = 0; j < JPW; ++j) {
        const size_t oi = obase + (size_t)t * ostride + 16 * (JPW * wave + j) + 4 * g4;
        if (p.out_bf16) {
          typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
          const bf16x4 o4 = {(__bf16)acc[j][0], (__bf16)acc[j][1], (__bf16)acc[j][2], (__bf16)acc[j][3]};
          *reinterpret_cast<bf16x4 *>(static_cast<__bf16 *>(p.o) + oi) = o4;
        } else {
          *reinterpret_cast<f32x4 *>(static_cast<float *>(p.o) + oi) = acc[j];
        }
      }
    }
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
