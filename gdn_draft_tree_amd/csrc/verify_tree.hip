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
// Work decomposition: one workgroup of d / 16 waves per (layer, request, head), wave w owning
// value channels [16 w, 16 w + 16); two workgroups per CU at d = 128 (16 waves per CU).
// Per head:
//  0. q, k, v rows go straight from HBM into LDS (buffer loads to LDS) and each wave loads
//     its S0 operand fragments into registers.  Wave 0 owns the per-node tree work (lane l
//     handles node l + 1): from its own early loads it checks the links, finds each node's
//     ancestors in its bitmask and forms the path gate g_t while the bulk loads are in flight;
//  1. every wave: P_Q = Q S0 and P_K = K S0 for its channels on MFMA (rows exact in bf16),
//     the C tiles kept in registers; the Gram tiles [Q; K] K^T of the lower node triangle on
//     MFMA, dealt over the waves, keeping the entries of ancestor pairs compactly by the depth
//     of the ancestor;
//  2. wave 0: one lane per node solves its path system and writes the node's W1 row (hi +
//     lo bf16) to LDS; every wave: V' = V - g P_K for its channels (V enters the C tiles
//     through a product with a 0/1 selector, so no transposed read of V is needed);
//  3. every wave: o^T = g P_Q^T + V'^T W1^T on MFMA (the C layout of V' is exactly the
//     operand layout the product needs), then the stores.
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
  // W1 row stride in bf16 elements: 16 rows read at one column start in distinct banks
  static constexpr int SPW = SP + 8;
  static constexpr int W1B = 2 * RM * SPW * 2;         // W1 rows, hi and lo bf16
  alignas(16) unsigned char qk[2 * ROWB];  // q rows, k rows
  alignas(16) uint16_t w1[W1B / 2];        // W1 rows: hi, then lo
  alignas(16) float lc[RM * kAR];      // k_t . k_s for s a strict ancestor of t, at depth(s)
  alignas(16) float mc[RM * kAR];      // q_t . k_s for s an ancestor-or-self of t, at depth(s)
  alignas(16) unsigned long long mask[RM];
  alignas(16) float gamma[16 * NT];    // path gate; zero past the node count
  float beta[RM];                      // b per node
  float cwl[kMaxAnc][64];              // wave 0's W1 weights, per depth and lane
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

// 16 x 16 x 16 product on bf16 bit patterns: lane l holds A[l % 16][4 (l / 16) + 0..3] and
// B[4 (l / 16) + 0..3][l % 16].
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4 mfma16(s16x4 a, s16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ short bf16_bits(float x) { return __builtin_bit_cast(short, (__bf16)x); }

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

__device__ __forceinline__ float bperm_f32(int lane_src, float x) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(lane_src << 2, __float_as_int(x)));
}
__device__ __forceinline__ float to_f32(uint16_t x) { return bf16_bits_to_f32(x); }
__device__ __forceinline__ float to_f32(float x) { return x; }

// S0LO: S0 enters the products as hi + lo bf16 (fp32 outputs); without it S0 is rounded to
// bf16 once, which for bf16 outputs stays below the outputs' own rounding.
template <int D, bool BF16IN, int NT, bool S0LO>
__global__ __launch_bounds__(4 * D, (BF16IN && !S0LO ? 2 : 1) * D / 64) void verify_kernel(VerifyParams p) {
  typedef VerifySmem<D, BF16IN, NT> SM;
  typedef typename SM::T T;
  constexpr int RM = SM::RM, SP = SM::SP, SPW = SM::SPW;
  constexpr int CH = 16 / (int)sizeof(T), CPR = D / CH;
  constexpr int KS = D / 32;               // MFMA k-steps over d_k
  constexpr int KSS = SP / 32;             // MFMA k-steps over the node axis
  constexpr int NW = D / 16;               // waves, one 16-channel value tile each
  constexpr int NTH = 64 * NW;             // threads
  constexpr int QMAX = SM::ROWB / 1024;    // 1 KiB row chunks per matrix
  constexpr int CPWQK = (2 * QMAX + NW - 1) / NW;  // q and k row chunks per wave
  constexpr int NS0 = KS * 2;              // S0 fragment loads per lane
  __shared__ SM s;

  const int tid = threadIdx.x, lane = tid & 63, g4 = lane >> 4, l16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int u = blockIdx.x;  // (layer, request, head)
  const int h = u % p.H, lb = u / p.H, b = lb % p.B;
  // n_nodes is read-only here: a scalar load
  const int32_t __attribute__((address_space(4))) *nn_c =
      (const int32_t __attribute__((address_space(4))) *)p.n_nodes;
  const int n = nn_c[b];
  if (n < 1 || n > p.R) return;  // no output for a request with an impossible node count
  const int nl = n - 1;
  const int ntl = (n + 15) / 16;  // node tiles in use
  const size_t rowbase = (size_t)lb * p.R;
  const size_t rstride = (size_t)p.H * D;  // elements between consecutive slots of one head
  const T *qrow = reinterpret_cast<const T *>(s.qk);
  const T *krow = reinterpret_cast<const T *>(s.qk + SM::ROWB);
  uint16_t *w1h = s.w1;
  uint16_t *w1l = w1h + RM * SPW;

  // ---- 0. loads ----------------------------------------------------------------------
  // Constant LDS stores first: issued before any load into LDS, they never wait for one.
  static_assert(RM * kAR / 4 <= 2 * NTH, "compact Gram rows: two stores per thread");
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int i = tid + NTH * x;
    if (i < RM * kAR / 4) {
      reinterpret_cast<float4 *>(s.lc)[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      reinterpret_cast<float4 *>(s.mc)[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  static_assert(SM::W1B % 16 == 0, "W1 in 16-byte stores");
#pragma unroll
  for (int x = 0; x < (SM::W1B / 16 + NTH - 1) / NTH; ++x) {
    const int i = tid + NTH * x;
    if (i < SM::W1B / 16) reinterpret_cast<uint4 *>(s.w1)[i] = make_uint4(0u, 0u, 0u, 0u);
  }
  if (tid >= n && tid < 16 * NT) s.gamma[tid] = 0.f;
  if (tid == 0) s.bad = 0;
  // Wave 0 owns the per-node tree work: lane l handles node t = l + 1 (the root is trivial)
  // and holds the gates of slot l for the other lanes.  These small loads go first, so wave 0
  // can wait for them alone (memory counters complete in order) and finish its per-node
  // prologue while the bulk loads below are still in flight.  All loads are unconditional at
  // clamped slots, so no branch forces an early wait and the counters stay static.
  const int t_me = lane + 1;
  const size_t tb = (size_t)b * p.R;
  const int tn = min(t_me, nl), ts = min(lane, nl);
  const unsigned long long w_mask = p.anc[tb + tn];
  const int w_par = p.parent[tb + tn];
  const T w_a0 = static_cast<const T *>(p.alpha)[(rowbase + ts) * p.H + h];
  const T w_b0 = static_cast<const T *>(p.beta)[(rowbase + ts) * p.H + h];
  const T w_a1 = static_cast<const T *>(p.alpha)[(rowbase + tn) * p.H + h];
  const T w_b1 = static_cast<const T *>(p.beta)[(rowbase + tn) * p.H + h];
  const unsigned long long my_mask = p.anc[tb + min(tid, nl)];  // -> LDS for the Gram scatter
  // Bulk loads in the order they are needed: q and k rows (the Gram tiles and the path solve
  // start on them alone), this wave's S0 fragments, then its v fragments (needed last).
  // q and k rows go straight into LDS: each wave instruction fills 64 consecutive 16-byte chunks; lane
  // l of chunk qi holds physical chunk 64 qi + l and fetches the logical chunk that the
  // swizzle places there.  Rows past the node count fetch row n-1 (never used).  Every wave
  // issues the same number of loads (its last chunk repeated, rewriting the same bytes).
  const T *gq = static_cast<const T *>(p.q) + (rowbase * p.H + h) * (size_t)D;
  const T *gk = static_cast<const T *>(p.k) + (rowbase * p.H + h) * (size_t)D;
  const T *gv = static_cast<const T *>(p.v) + (rowbase * p.H + h) * (size_t)D;
  const int nb = (int)(n * rstride * sizeof(T));
  auto row_chunk = [&](const __amdgpu_buffer_rsrc_t &rs, unsigned char *mat_lds, int qi) {
    const int pc = 64 * qi + lane, r = pc / CPR, c = (pc % CPR) ^ (r & (CPR - 1));
    const unsigned off = (unsigned)((min(r, nl) * (int)rstride + c * CH) * (int)sizeof(T));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t *)(mat_lds + 1024 * qi), 16, off, 0, 0, 0);
  };
  __builtin_amdgcn_sched_barrier(0);
  {
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc((void *)gq, 0, nb, 0x00020000);
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void *)gk, 0, nb, 0x00020000);
#pragma unroll
    for (int x = 0; x < CPWQK; ++x) {
      const int item = min(wave + NW * x, 2 * QMAX - 1);
      if (item < QMAX)
        row_chunk(rq, s.qk, item);
      else
        row_chunk(rk, s.qk + SM::ROWB, item - QMAX);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  // S0 operand fragments of this wave's value channels: lane (g, c) holds
  // S0[32 ks + 8 g + 0..7][channel 16 wave + c], contiguous in the [d_v][d_k] state layout.
  f32x4 s0r[KS][2];
  {
    const float *sr = p.state + ((size_t)u * D + 16 * wave + l16) * D + 8 * g4;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s0r[ks][0] = *reinterpret_cast<const f32x4 *>(sr + 32 * ks);
      s0r[ks][1] = *reinterpret_cast<const f32x4 *>(sr + 32 * ks + 4);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  // v fragments of this wave's 16 channels, the A operand of a 16 x 16 x 16 product: lane
  // (g, r) holds V[16 mt + r][16 wave + 4 g + 0..3].  Rows past the node count lie beyond the
  // buffer's range and read as zero.
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  typename std::conditional<BF16IN, u32x2, u32x4>::type vld[NT];
  {
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void *)gv, 0, nb, 0x00020000);
#pragma unroll
    for (int mt = 0; mt < NT; ++mt) {
      const int off = ((16 * mt + l16) * (int)rstride + 16 * wave + 4 * g4) * (int)sizeof(T);
      if constexpr (BF16IN)
        vld[mt] = __builtin_amdgcn_raw_buffer_load_b64(rv, off, 0, 0);
      else
        vld[mt] = __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  if (tid < n) s.mask[tid] = my_mask;

  // ---- 0b. wave 0, per node: link check, ancestors by depth, path gate, W1 weights -------
  uint32_t ancw[5] = {0u, 0u, 0u, 0u, 0u};  // slot of the ancestor at depth e, byte e
  int d_me = 0;
  if (wave == 0) {
    const bool tv = t_me < n;
    const float a0 = to_f32(w_a0), b0 = to_f32(w_b0), a1 = to_f32(w_a1), b1 = to_f32(w_b1);
    const unsigned long long m = w_mask;
    d_me = __popcll(m);
    // the parent's mask is the node mask held by lane parent - 1 (the root's mask is zero)
    const int pl = min(max(w_par - 1, 0), 63);
    const uint32_t pm_lo = (uint32_t)__builtin_amdgcn_ds_bpermute(pl << 2, (int)(uint32_t)m);
    const uint32_t pm_hi = (uint32_t)__builtin_amdgcn_ds_bpermute(pl << 2, (int)(uint32_t)(m >> 32));
    const unsigned long long pm = w_par == 0 ? 0ull : (((unsigned long long)pm_hi << 32) | pm_lo);
    const bool ok = d_me <= kMaxP && w_par >= 0 && w_par < t_me && m == (pm | (1ull << (t_me - 1)));
    if (tv && !ok) s.bad = 1;
    d_me = min(d_me, kMaxP);
    float bet[kMaxAnc], alp[kMaxAnc];  // b and a of the ancestor at depth e
    alp[0] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a0), 0));
    bet[0] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(b0), 0));
    float g = alp[0];
    unsigned long long mm = m;
#pragma unroll
    for (int e = 1; e <= kMaxP; ++e) {
      const int a = min(__ffsll((long long)mm), nl);  // 0 (the root) beyond the depth
      mm &= mm - 1;
      ancw[e >> 2] |= (uint32_t)a << (8 * (e & 3));
      // gates of slot a: held by lane a, except t itself (slot 64 has no lane)
      float av = bperm_f32(a, a0), bv = bperm_f32(a, b0);
      if (a == t_me) { av = a1; bv = b1; }
      alp[e] = av;
      bet[e] = bv;
      g *= (e <= d_me) ? av : 1.f;
    }
    // W1[t, anc e] = cw[e] z[e] with cw[e] = b_{anc e} g_t / g_{anc e}
    float rr = 1.f;
#pragma unroll
    for (int e = kMaxP; e >= 0; --e) {
      s.cwl[e][lane] = (e <= d_me) ? rr * bet[e] : 0.f;
      rr *= (e <= d_me) ? alp[e] : 1.f;
    }
    if (tv) {
      s.gamma[t_me] = g;
      s.beta[t_me] = b1;
    }
    if (lane == 0) {
      s.gamma[0] = alp[0];
      s.beta[0] = bet[0];
    }
  }
  // q and k rows have landed; S0 and v may still be in flight
  constexpr int kAfterQK = NS0 + NT;
  static_assert(kAfterQK < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0070 | ((kAfterQK & 15) | ((kAfterQK >> 4) << 14)));  // vmcnt(..) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();

  // ---- 1. Gram tiles [Q; K] K^T of the lower node triangle, dealt over the waves ----------
  // Tile pair i = mt (mt + 1) / 2 + nt goes to wave NW - 1 - i % NW (wave 0, which has the
  // path solve next, gets the fewest).  Transposed: lane (g, t) owns node t = 16 mt + l16 and
  // gets k_s . k_t and k_s . q_t for s = 16 nt + 4 g + 0..3.  Entries of ancestor pairs are
  // kept at depth(s) = (t's ancestors-or-self in slots 0..s) - 1 (the k.k ones times b_t, the
  // factor the path solve applies); the rest go to padding entries 17..19.
  if (wave == 1 && lane == 0 && s.mask[0] != 0ull) s.bad = 1;  // the root has no ancestors
#pragma unroll
  for (int mt = 0; mt < NT; ++mt) {
#pragma unroll
    for (int nt = 0; nt <= mt; ++nt) {
      if (wave != NW - 1 - (mt * (mt + 1) / 2 + nt) % NW || mt >= ntl) continue;
      // Row fragments are read at the tile's rows as they are: rows past the node count hold
      // finite values (copies of the last row, or the next LDS region), and the entries they
      // produce are never kept.
      const int tme = 16 * mt + l16, ra = min(tme, nl);
      const int rb = 16 * nt + l16;
      f32x4 gk4 = {0.f, 0.f, 0.f, 0.f}, gq4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        bf16x8 aqh, aql, akh, akl, bh, bl;
        row_frag<D, BF16IN>(qrow, tme, 32 * ks + 8 * g4, aqh, aql);
        row_frag<D, BF16IN>(krow, tme, 32 * ks + 8 * g4, akh, akl);
        row_frag<D, BF16IN>(krow, rb, 32 * ks + 8 * g4, bh, bl);
        gk4 = mfma(bh, akh, gk4);
        gq4 = mfma(bh, aqh, gq4);
        if constexpr (!BF16IN) {
          gk4 = mfma(bl, akh, gk4);
          gk4 = mfma(bh, akl, gk4);
          gq4 = mfma(bl, aqh, gq4);
          gq4 = mfma(bh, aql, gq4);
        }
      }
      const unsigned long long tmask = s.mask[ra];
      const unsigned long long aset = (tmask << 1) | 1ull;  // slot s <= 63 -> bit s; root in
      const float bt = s.beta[ra];
      const int trow = ra * kAR;
      const bool rowok = tme < n;
      const int sn0 = 16 * nt + 4 * g4;
      uint32_t bits;  // ancestor flags of slots sn0 .. sn0 + 3
      int cbelow;     // t's ancestors-or-self in slots 0 .. sn0 - 1
      if (nt < 4) {
        bits = (uint32_t)(aset >> sn0) & 0xfu;
        cbelow = __popcll(aset & ((1ull << sn0) - 1ull));
      } else {  // slots 64..79: only slot 64, and only as t itself
        bits = (g4 == 0) ? (uint32_t)(tmask >> 63) : 0u;
        cbelow = __popcll(aset);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int sn = sn0 + r;
        const int es = cbelow + __popc(bits & ((2u << r) - 1u)) - 1;
        const bool keep = rowok && ((bits >> r) & 1u) && sn <= tme && es <= kMaxP;
        const int dummy = trow + kMaxAnc + (r % 3);
        s.mc[keep ? trow + es : dummy] = gq4[r];
        s.lc[keep && sn != tme ? trow + es : dummy] = gk4[r] * bt;
      }
    }
  }
  lds_barrier();

  // ---- 2. wave 0: path solve, one lane per node, and its W1 row (overlapping the S0 loads);
  //         every wave: P_Q = Q S0 and P_K = K S0 for its channels on MFMA, and V' -----------
  if (wave == 0) {
    const bool tv = t_me < n;
    const int t = tn;
    const int dmax = wave_max_i32(tv ? d_me : 0);
    auto anc_at = [&](int e) -> int { return (int)((ancw[e >> 2] >> (8 * (e & 3))) & 0xffu); };
    float z[kAR];  // right-hand side q_t . k_{anc e}; zero beyond the depth
#pragma unroll
    for (int v = 0; v < kAR / 4; ++v) {
      const float4 x = reinterpret_cast<const float4 *>(&s.mc[t * kAR])[v];
      z[4 * v] = x.x; z[4 * v + 1] = x.y; z[4 * v + 2] = x.z; z[4 * v + 3] = x.w;
    }
    // deepest ancestor first, two steps per group with the group's rows loaded together.
    // Beyond a lane's depth z is zero and the ancestor slot is the root, so those steps
    // change nothing; groups deeper than every lane are skipped.
#pragma unroll
    for (int grp = kMaxP / 2 - 1; grp >= 0; --grp) {
      if (2 * grp + 1 > dmax) continue;
      float4 rw[2][4];
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int e2 = 2 * grp + 2 - r;
        const float4 *row = reinterpret_cast<const float4 *>(&s.lc[anc_at(e2) * kAR]);
#pragma unroll
        for (int v = 0; v < (e2 + 3) / 4; ++v) rw[r][v] = row[v];
      }
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int e2 = 2 * grp + 2 - r;
        const float c = z[e2];  // the b of the step is folded into the stored k.k entries
#pragma unroll
        for (int v = 0; v < (e2 + 3) / 4; ++v) {
          const float xs[4] = {rw[r][v].x, rw[r][v].y, rw[r][v].z, rw[r][v].w};
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (4 * v + i < e2) z[4 * v + i] -= c * xs[i];
        }
      }
    }
    // W1[t, anc e] = cw[e] z[e] into the (cleared) dense row, hi + lo bf16
    if (tv) {
#pragma unroll
      for (int e = 0; e <= kMaxP; ++e) {
        if (e <= d_me) {
          const float w = s.cwl[e][lane] * z[e];
          const __bf16 hv = (__bf16)w;
          const __bf16 lv = (__bf16)(w - (float)hv);
          const int pos = t * SPW + w1_pos(anc_at(e));
          w1h[pos] = __builtin_bit_cast(uint16_t, hv);
          w1l[pos] = __builtin_bit_cast(uint16_t, lv);
        }
      }
    }
  } else if (wave == 1 && lane == 0) {
    // the root: W1[0, 0] = b_0 (q_0 . k_0)
    const float w = s.beta[0] * s.mc[0];
    const __bf16 hv = (__bf16)w;
    w1h[0] = __builtin_bit_cast(uint16_t, hv);
    w1l[0] = __builtin_bit_cast(uint16_t, (__bf16)(w - (float)hv));
  }
  bf16x8 s0h[KS], s0l[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const float x[8] = {s0r[ks][0][0], s0r[ks][0][1], s0r[ks][0][2], s0r[ks][0][3],
                        s0r[ks][1][0], s0r[ks][1][1], s0r[ks][1][2], s0r[ks][1][3]};
    if constexpr (S0LO) {
      split8(x, s0h[ks], s0l[ks]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) s0h[ks][e] = (__bf16)x[e];
    }
  }
  // P_Q is kept transposed (lane (g, t) holds P_Q[t][16 wave + 4 g + 0..3]: the C layout of
  // S0^T Q^T), P_K node-major (lane (g, c) holds P_K[4 g + 0..3][16 wave + c]).  Both come
  // from the same registers: the S0 fragments are the A operand of one product and the B
  // operand of the other, and so are the row fragments.
  f32x4 pqt[NT], pk[NT];  // tiles past the node count are never read
#pragma unroll
  for (int mt = 0; mt < NT; ++mt) {
    if (mt >= ntl) continue;
    const int ra = 16 * mt + l16;  // rows past the node count: finite, never used
    pqt[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    pk[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8 aqh, aql, akh, akl;
      row_frag<D, BF16IN>(qrow, ra, 32 * ks + 8 * g4, aqh, aql);
      row_frag<D, BF16IN>(krow, ra, 32 * ks + 8 * g4, akh, akl);
      pqt[mt] = mfma(s0h[ks], aqh, pqt[mt]);
      pk[mt] = mfma(akh, s0h[ks], pk[mt]);
      if constexpr (S0LO) {
        pqt[mt] = mfma(s0l[ks], aqh, pqt[mt]);
        pk[mt] = mfma(akh, s0l[ks], pk[mt]);
      }
      if constexpr (!BF16IN) {
        pqt[mt] = mfma(s0h[ks], aql, pqt[mt]);
        pk[mt] = mfma(akl, s0h[ks], pk[mt]);
      }
    }
  }
  // V' = V - g P_K for this wave's channels.  V enters the C tiles (lane (g, c): rows 4 g +
  // 0..3 of channel c) through a product with the identity, and the result is packed as hi +
  // lo bf16, the A operand of V'^T W1^T.
  bf16x8 vph[KSS], vpl[KSS];
  {
    s16x4 ident;
#pragma unroll
    for (int e = 0; e < 4; ++e) ident[e] = (short)((4 * g4 + e == l16) ? 0x3f80 : 0);  // bf16 1
#pragma unroll
    for (int mt = 0; mt < 2 * KSS; ++mt) {
      f32x4 vp = {0.f, 0.f, 0.f, 0.f};
      if (mt < NT && mt < ntl) {
        const int mc_ = mt < NT ? mt : NT - 1;  // (static index; mt < NT here)
        const float4 gm = *reinterpret_cast<const float4 *>(&s.gamma[16 * mt + 4 * g4]);
        vp[0] = -gm.x * pk[mc_][0];
        vp[1] = -gm.y * pk[mc_][1];
        vp[2] = -gm.z * pk[mc_][2];
        vp[3] = -gm.w * pk[mc_][3];
        if constexpr (BF16IN) {
          vp = mfma16(__builtin_bit_cast(s16x4, vld[mc_]), ident, vp);
        } else {
          const f32x4 x = __builtin_bit_cast(f32x4, vld[mc_]);
          s16x4 vh, vl;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const __bf16 hv = (__bf16)x[i];
            vh[i] = __builtin_bit_cast(short, hv);
            vl[i] = bf16_bits(x[i] - (float)hv);
          }
          vp = mfma16(vh, ident, vp);
          vp = mfma16(vl, ident, vp);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const __bf16 hv = (__bf16)vp[i];
        vph[mt >> 1][4 * (mt & 1) + i] = hv;
        vpl[mt >> 1][4 * (mt & 1) + i] = (__bf16)(vp[i] - (float)hv);
      }
    }
  }
  // W1 is complete
  lds_barrier();
  const bool bad = s.bad != 0;

  // ---- 3. o^T = g P_Q^T + V'^T W1^T for this wave's value channels, node tile by node tile --
  // A operand: V' (its registers are exactly the A layout of V'^T), B operand: W1 rows from
  // LDS; W1 is zero above the diagonal, so node chunks past the tile are skipped.  Lane
  // (g, t) ends with o[t][16 wave + 4 g + 0..3]: one 8-byte (bf16) store per tile, through a
  // buffer whose range ends at the last node, so rows past the node count are dropped.  An
  // inconsistent tree gives NaN outputs.
  {
    const int oes = p.out_bf16 ? 2 : 4;
    const unsigned ostride = (unsigned)(p.H * D * oes);
    char *obase = static_cast<char *>(p.o) + (rowbase * p.H + h) * (size_t)D * oes;
    const int orange = (nl * p.H * D + D) * oes;
    const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(obase, 0, orange, 0x00020000);
#pragma unroll
    for (int mt = 0; mt < NT; ++mt) {
      if (mt >= ntl) break;
      const int t = 16 * mt + l16, tr = t;  // W1 rows past the node count: never stored
      const float gt = s.gamma[t];
      f32x4 acc = gt * pqt[mt];
#pragma unroll
      for (int kk = 0; kk < KSS; ++kk) {
        if (32 * kk > 16 * mt + 15) break;
        const bf16x8 wh = frag16(w1h + tr * SPW + 32 * kk + 8 * g4);
        const bf16x8 wl = frag16(w1l + tr * SPW + 32 * kk + 8 * g4);
        acc = mfma(vph[kk], wh, acc);
        acc = mfma(vpl[kk], wh, acc);
        acc = mfma(vph[kk], wl, acc);
      }
      if (bad) acc = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
      const unsigned vo = (unsigned)t * ostride + (unsigned)((16 * wave + 4 * g4) * oes);
      if (p.out_bf16) {
        const uint32_t lo = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)acc[0]) |
                            ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)acc[1]) << 16);
        const uint32_t hi = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)acc[2]) |
                            ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)acc[3]) << 16);
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{lo, hi}, ro, (int)vo, 0, 0);
      } else {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc), ro, (int)vo, 0, 0);
      }
    }
  }
}

template <int D, bool BF16IN, int NT>
hipError_t launch_one(const VerifyParams &p, hipStream_t stream) {
  const unsigned units = (unsigned)(p.L * p.B * p.H);
  if constexpr (BF16IN) {
    if (p.out_bf16) {
      hipLaunchKernelGGL((verify_kernel<D, true, NT, false>), dim3(units), dim3(4 * D), 0, stream, p);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((verify_kernel<D, BF16IN, NT, true>), dim3(units), dim3(4 * D), 0, stream, p);
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
