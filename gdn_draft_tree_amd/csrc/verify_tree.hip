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
// k_s u_s^T over the ancestors-or-self s of t, with pseudo-values u that solve a system
// triangular along root paths.  Scaling the unknowns by the path gates removes every gate
// from that system: for node t with ancestors-or-self anc e at depths e = 0..d_t, let z
// solve (deepest first)
//     z[e] + sum_{e2 > e} z[e2] b_{anc e2} (k_{anc e2} . k_{anc e}) = q_t . k_{anc e}.
// With Y[t, anc e] = b_{anc e} z[e] and W1[t, anc e] = (g_t / g_{anc e}) Y[t, anc e],
//     o_t = S0^T E_t + sum_s W1[t, s] v_s,     E_t = g_t (q_t - sum_s Y[t, s] k_s).
// So the committed state S0, the only large operand (d_k x d_v fp32), enters through ONE
// dense product S0^T E, and the tree enters through small work that needs q, k, a and b
// only: Gram entries of ancestor pairs, one path solve per node, and the "effective
// queries" E.  Y and W1 are bounded by one in magnitude when |q| = |k| = 1 and a, b lie in
// [0, 1] (W1[t, s] is the coefficient of v_s in o_t, and z does not depend on the gates).
//
// Work decomposition: one workgroup per (layer, request, head) with two kinds of waves.
//  * d/16 product waves, wave w owning value channels [16 w, 16 w + 16): they only stream
//    this head's committed state and v rows into registers, form V^T W1^T once W1 is in
//    LDS, convert the state to fp16 as it lands, and once E is in LDS add S0^T E^T.
//  * four tree waves: wave 0 loads the per-node inputs and does the per-node prologue; waves
//    1..3 stream the q and k rows into LDS (buffer loads to LDS).  Together they compute the
//    Gram tiles [Q; K] K^T of the lower node triangle, then wave 0 does the per-node path
//    solves (one lane per node) that give Y and W1, and all four form E on MFMA.  They order
//    their phases through an LDS counter.
// A first workgroup barrier orders the loads (below); three more hand over W1, then E, then
// the finished output rows, which are staged in LDS and stored as whole rows by every wave.
// A product wave that issues its
// state loads stalls until the memory pipeline accepts them, so the waves that carry the
// latency-bound tree work issue only the small row loads, ahead of the state (and run at
// raised priority).  When the state lands, only one dense product and the stores remain.
//
// Precision: MFMA operands are fp16 with fp32 accumulation.  Rows in bf16 convert to fp16
// exactly; the state and v columns of a product wave are scaled by one power of two (from
// their largest magnitude) before the conversion and the outputs are scaled back, so the
// fp16 range holds for any state scale.  The Gram entries are exact for bf16 rows (fp32
// inputs enter the Gram as hi + lo bf16 pairs), and the path solve runs in fp32.

#include <type_traits>

#include "gdntree_internal.h"

namespace gdntree {
namespace {

constexpr int kAR = 20;  // compact row: ancestor depths 0..16, padded to five 16-byte vectors
constexpr int kLdsBytes = 160 * 1024;

template <bool BF16IN>
struct InT;
template <>
struct InT<true> { typedef uint16_t T; };
template <>
struct InT<false> { typedef float T; };

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

template <int D, bool BF16IN, int NT>
struct VerifySmem {
  typedef typename InT<BF16IN>::T T;
  static constexpr int RM = (16 * NT < kMaxSlots) ? 16 * NT : kMaxSlots;  // node rows held
  static constexpr int ROWB = (RM * D * (int)sizeof(T) + 1023) / 1024 * 1024;  // whole 1 KiB loads
  static constexpr int SP = (16 * NT + 31) / 32 * 32;  // node (contraction) axis of Y K and W1 V
  // Y / W1 row stride in fp16 elements: 16 rows read at one column start hit distinct banks
  static constexpr int SPW = SP + 8;
  // fp16 rows of E: in place of the q rows for bf16 inputs, a region of their own for fp32
  static constexpr int EB = BF16IN ? 16 : (RM * D * 2 + 15) / 16 * 16;
  alignas(16) unsigned char qk[2 * ROWB];  // q rows (then E for bf16 inputs), k rows
  alignas(16) unsigned char e16[EB];
  alignas(16) _Float16 y[RM * SPW];        // Y rows, the node axis in the MFMA k order
  alignas(16) _Float16 w1[RM * SPW];       // W1 rows, same layout
  alignas(16) float lc[RM * kAR];          // b_t k_t . k_s for s a strict ancestor of t, at depth(s)
  alignas(16) float mc[RM * kAR];          // q_t . k_s for s an ancestor-or-self of t, at depth(s)
  alignas(16) unsigned long long mask[RM];
  alignas(16) float gamma[16 * NT];        // path gate
  float beta[RM];                          // b per node
  float cwl[kMaxAnc][64];                  // W1 weights b_{anc e} g_t / g_{anc e}, per depth and lane
  int bad;
  int sync;                                // tree-wave phase counter
};

constexpr int kTreeWaves = 4;

template <int D, bool BF16IN, int NT>
struct VerifyShape {
  static constexpr int NW = D / 16;        // product waves
  static constexpr int WAVES = NW + kTreeWaves;
  static constexpr int NTH = 64 * WAVES;
  static constexpr int LDS = (int)sizeof(VerifySmem<D, BF16IN, NT>);
  static constexpr int WG_PER_CU0 = kLdsBytes / LDS < 1 ? 1 : kLdsBytes / LDS;
  static constexpr int WG_PER_CU = WG_PER_CU0 < 2 ? WG_PER_CU0 : 2;
  // A workgroup's waves are dealt over the CU's four SIMDs, so the register budget must let
  // every SIMD hold ceil(WAVES / 4) waves of each resident workgroup.
  static constexpr int WPEU = WG_PER_CU * ((WAVES + 3) / 4);
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
__device__ __forceinline__ f16x8 hfrag(const void *p) {
  return __builtin_bit_cast(f16x8, *reinterpret_cast<const uint4 *>(p));
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

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
// 16 x 16 x 16: lane l holds A[l % 16][4 (l / 16) + 0..3] and B[4 (l / 16) + 0..3][l % 16].
__device__ __forceinline__ f32x4 mfma16_f16(f16x4 a, f16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

// Eight consecutive elements of one LDS row (a 16-byte chunk for bf16, two for fp32): the
// operand fragment of a Gram product that contracts over d.
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

// Four consecutive elements of one LDS row as fp32 (col is a multiple of 4).
template <int D, bool BF16IN>
__device__ __forceinline__ f32x4 row4(const typename InT<BF16IN>::T *rows, int r, int col) {
  if constexpr (BF16IN) {
    const uint2 x = *reinterpret_cast<const uint2 *>(rows + swz<D, 8>(r, col));
    return f32x4{__uint_as_float(x.x << 16), __uint_as_float(x.x & 0xffff0000u),
                 __uint_as_float(x.y << 16), __uint_as_float(x.y & 0xffff0000u)};
  } else {
    const float4 x = *reinterpret_cast<const float4 *>(rows + swz<D, 4>(r, col));
    return f32x4{x.x, x.y, x.z, x.w};
  }
}

// Position of node s inside its 32-node chunk of a Y / W1 row.  The A operand of Y K and
// V^T W1^T holds, in lane (g, c), nodes 4 g + 0..3 of the chunk's first 16-node tile and
// 16 + 4 g + 0..3 of its second (the C layout of two products with the identity), so the k
// index 8 g + e of the product stands for node 4 g + e (e < 4) or 16 + 4 g + e - 4 (e >= 4);
// the rows are stored in that k order.
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

__device__ __forceinline__ float bperm_f32(int lane_src, float x) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(lane_src << 2, __float_as_int(x)));
}
__device__ __forceinline__ float to_f32(uint16_t x) { return bf16_bits_to_f32(x); }
__device__ __forceinline__ float to_f32(float x) { return x; }

// The tree waves meet here: each finishes its own memory work (loads into LDS included),
// counts itself in, and waits for the others.  The wait is bounded; a wave that
// gives up marks the request bad (NaN outputs) instead of hanging.
__device__ __forceinline__ void tree_sync(int *cnt, int *bad, int target, int lane) {
  __builtin_amdgcn_s_waitcnt(0);  // vmcnt(0) expcnt(0) lgkmcnt(0)
  if (lane == 0) __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
  int spins = 0;
  while (__hip_atomic_load(cnt, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < target) {
    __builtin_amdgcn_s_sleep(1);
    if (++spins > (1 << 22)) {
      *bad = 1;
      break;
    }
  }
}

// Output rows of one head, staged in LDS with swizzled 16-byte chunks, stored as whole rows
// (16-byte pieces, consecutive lanes along a row) by every wave of the workgroup.
template <int D>
__device__ __forceinline__ void store_rows(const VerifyParams &p, const unsigned char *stage, int n,
                                           size_t rowbase, int h, int tid, int nth) {
  const int oes = p.out_bf16 ? 2 : 4;
  const int cpr = D * oes / 16;  // 16-byte chunks per row: a power of two
  const unsigned ostride = (unsigned)(p.H * D * oes);
  char *obase = static_cast<char *>(p.o) + (rowbase * p.H + h) * (size_t)D * oes;
  const int orange = ((n - 1) * p.H * D + D) * oes;
  const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(obase, 0, orange, 0x00020000);
  for (int c = tid; c < n * cpr; c += nth) {
    const int r = c / cpr, lc = c % cpr;
    const u32x4 x = *reinterpret_cast<const u32x4 *>(stage + 16 * (r * cpr + (lc ^ (r & (cpr - 1)))));
    __builtin_amdgcn_raw_buffer_store_b128(x, ro, (int)((unsigned)r * ostride + 16u * lc), 0, 0);
  }
}

template <int D, bool BF16IN, int NT>
__global__ __launch_bounds__((VerifyShape<D, BF16IN, NT>::NTH), (VerifyShape<D, BF16IN, NT>::WPEU))
void verify_kernel(VerifyParams p) {
  typedef VerifySmem<D, BF16IN, NT> SM;
  typedef typename SM::T T;
  constexpr int RM = SM::RM, SPW = SM::SPW;
  constexpr int CH = 16 / (int)sizeof(T), CPR = D / CH;
  constexpr int KS = D / 32;               // MFMA k-steps over d_k
  constexpr int KSS = SM::SP / 32;         // MFMA k-steps over the node axis
  constexpr int NW = D / 16;               // product waves; also the channel tiles of E
  constexpr int QMAX = SM::ROWB / 1024;    // 1 KiB row chunks per matrix
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
  const int nb = (int)(n * rstride * sizeof(T));  // byte range of this head's used rows
  // fp16 rows of E (same swizzled layout as bf16 rows)
  _Float16 *erow = reinterpret_cast<_Float16 *>(BF16IN ? s.qk : s.e16);
  // Output rows are staged from the k rows on: once E is formed nothing reads the k rows, Y,
  // W1 or the compact Gram rows again.
  unsigned char *ostage = s.qk + SM::ROWB;
  static_assert(offsetof(SM, mask) - SM::ROWB >= (size_t)SM::RM * D * 4, "output staging fits");

  if (wave < NW) {
    // ================================ product waves ==================================
    // The tree waves issue their row loads before this barrier, so they are queued ahead of
    // the state loads below.
    __builtin_amdgcn_s_barrier();
    const T *gv = static_cast<const T *>(p.v) + (rowbase * p.H + h) * (size_t)D;
    // v fragments, the A operand of a 16 x 16 x 16 product: lane (g, r) holds V[16 mt + r]
    // [16 wave + 4 g + 0..3].  Rows past the node count lie beyond the buffer's range and
    // read as zero.
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
    // state fragments of this wave's value channels, the A operand of S0^T E^T: lane (g, c)
    // holds S0[32 ks + 8 g + 0..7][channel 16 wave + c], contiguous in the [d_v][d_k] layout.
    f32x4 s0r[KS][2];
    {
      const float *sr = p.state + ((size_t)u * D + 16 * wave + l16) * D + 8 * g4;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s0r[ks][0] = *reinterpret_cast<const f32x4 *>(sr + 32 * ks);
        s0r[ks][1] = *reinterpret_cast<const f32x4 *>(sr + 32 * ks + 4);
      }
    }
    __builtin_amdgcn_s_barrier();  // (1) W1 is in LDS

    // ---- V^T W1^T for this wave's channels, before the state has landed ------------------
    // v is scaled by a power of two 2^-ev chosen from its largest magnitude (the scaled
    // values lie in [2^14, 2^15) at most), so the fp16 range holds for any v scale.
    float mv = 0.f;
#pragma unroll
    for (int mt = 0; mt < NT; ++mt) {
      if constexpr (BF16IN) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          mv = fmaxf(mv, fabsf(__uint_as_float(vld[mt][i] << 16)));
          mv = fmaxf(mv, fabsf(__uint_as_float(vld[mt][i] & 0xffff0000u)));
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) mv = fmaxf(mv, fabsf(__uint_as_float(vld[mt][i])));
      }
    }
    // non-negative floats order like their bit patterns; ex = clamped biased exponent
    const int exv = min(max((wave_max_i32(__float_as_int(mv)) >> 23) & 0xff, 15), 254);
    // V^T in the C layout (lane (g, c): rows 4 g + 0..3 of channel c) through a product with
    // the identity, packed as the A operand of V^T W1^T.
    f32x4 acc[NT];
    {
      f16x8 vph[KSS];
      f16x4 ident;
#pragma unroll
      for (int e = 0; e < 4; ++e) ident[e] = (_Float16)((4 * g4 + e == l16) ? 1.f : 0.f);
#pragma unroll
      for (int mt = 0; mt < 2 * KSS; ++mt) {
        f32x4 vp = {0.f, 0.f, 0.f, 0.f};
        if (mt < NT && mt < ntl) {
          const int mc_ = mt < NT ? mt : NT - 1;  // (static index; mt < NT here)
          f16x4 a;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float x;
            if constexpr (BF16IN)
              x = (i & 1) ? __uint_as_float(vld[mc_][i >> 1] & 0xffff0000u) : __uint_as_float(vld[mc_][i >> 1] << 16);
            else
              x = __uint_as_float(vld[mc_][i]);
            a[i] = (_Float16)__builtin_amdgcn_ldexpf(x, 141 - exv);
          }
          vp = mfma16_f16(a, ident, vp);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) vph[mt >> 1][4 * (mt & 1) + i] = (_Float16)vp[i];
      }
      // W1 is zero above the diagonal, so node chunks past the tile are skipped
#pragma unroll
      for (int mt = 0; mt < NT; ++mt) {
        acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (mt >= ntl) continue;
        const int t = 16 * mt + l16;
#pragma unroll
        for (int kk = 0; kk < KSS; ++kk) {
          if (32 * kk > 16 * mt + 15) break;
          acc[mt] = mfma_f16(vph[kk], hfrag(s.w1 + t * SPW + 32 * kk + 8 * g4), acc[mt]);
        }
      }
    }
    // The state, as soon as it has landed (before E is ready), is scaled by 2^(141 - ex) with
    // ex >= the v exponent, so both scaled operands stay inside the fp16 range; the V^T W1^T
    // part is rescaled to match (exact; nothing to do in the usual case ex == exv).
    float ms = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) ms = fmaxf(ms, fabsf(s0r[ks][j][i]));
    const int exs = min(max((wave_max_i32(__float_as_int(ms)) >> 23) & 0xff, 15), 254);
    const int ex = max(exs, exv);
    f16x8 s0h[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) s0h[ks][e] = (_Float16)__builtin_amdgcn_ldexpf(s0r[ks][e >> 2][e & 3], 141 - ex);
    if (ex != exv) {
#pragma unroll
      for (int mt = 0; mt < NT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[mt][i] = __builtin_amdgcn_ldexpf(acc[mt][i], exv - ex);
    }
    __builtin_amdgcn_s_barrier();  // (2) E is in LDS
    const bool bad = __builtin_amdgcn_readfirstlane(s.bad) != 0;

    // ---- + S0^T E^T ------------------------------------------------------------------------
    // Lane (g, t) ends with o[t][16 wave + 4 g + 0..3], written into the output rows staged in
    // LDS (rows past the node count are not written).  An inconsistent tree gives NaN outputs.
#pragma unroll
    for (int mt = 0; mt < NT; ++mt) {
      if (mt >= ntl) break;
      const int t = 16 * mt + l16;
      f32x4 o4 = acc[mt];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) o4 = mfma_f16(s0h[ks], hfrag(erow + swz<D, 8>(t, 32 * ks + 8 * g4)), o4);
#pragma unroll
      for (int i = 0; i < 4; ++i) o4[i] = __builtin_amdgcn_ldexpf(o4[i], ex - 141);
      if (bad) o4 = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
      if (t < n) {
        if (p.out_bf16) {
          const uint32_t lo = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)o4[0]) |
                              ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)o4[1]) << 16);
          const uint32_t hi = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)o4[2]) |
                              ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)o4[3]) << 16);
          *reinterpret_cast<u32x2 *>(ostage + 2 * swz<D, 8>(t, 16 * wave + 4 * g4)) = u32x2{lo, hi};
        } else {
          *reinterpret_cast<f32x4 *>(ostage + 4 * swz<D, 4>(t, 16 * wave + 4 * g4)) = o4;
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's output rows are staged
    __builtin_amdgcn_s_barrier();        // (3) every output row is staged
    store_rows<D>(p, ostage, n, rowbase, h, 64 * wave + lane, 64 * (NW + kTreeWaves));
    return;
  }

  // ================================== tree waves =====================================
  __builtin_amdgcn_s_setprio(3);
  const int tw = wave - NW;  // 0: per-node tree work and the path solves; 1..3: clears
  const T *qrow = reinterpret_cast<const T *>(s.qk);
  const T *krow = reinterpret_cast<const T *>(s.qk + SM::ROWB);
  const size_t tb = (size_t)b * p.R;
  // tw 0 issues only the small per-node loads: an LDS write of a wave waits for that wave's
  // own loads into LDS, and its prologue writes LDS early.  tw 1..3 clear Y, W1 (zero off the
  // ancestor pattern) and the compact Gram rows first, for the same reason, then load the q
  // and k rows.
  const int t_me = lane + 1;
  const int tn = min(t_me, nl);
  const int ts = min(lane, nl);
  unsigned long long w_mask = 0ull, my_mask = 0ull;
  int w_par = 0;
  uint32_t w_a0 = 0u, w_b0 = 0u, w_a1 = 0u, w_b1 = 0u;  // gate bits
  if (tw == 0) {
    if (lane == 0) {
      s.sync = 0;
      s.bad = 0;
    }
    w_mask = p.anc[tb + tn];
    w_par = p.parent[tb + tn];
    my_mask = p.anc[tb + ts];
    const T *ga = static_cast<const T *>(p.alpha), *gb = static_cast<const T *>(p.beta);
    if constexpr (BF16IN) {
      w_a0 = reinterpret_cast<const uint16_t *>(ga)[(rowbase + ts) * p.H + h];
      w_b0 = reinterpret_cast<const uint16_t *>(gb)[(rowbase + ts) * p.H + h];
      w_a1 = reinterpret_cast<const uint16_t *>(ga)[(rowbase + tn) * p.H + h];
      w_b1 = reinterpret_cast<const uint16_t *>(gb)[(rowbase + tn) * p.H + h];
    } else {
      w_a0 = reinterpret_cast<const uint32_t *>(ga)[(rowbase + ts) * p.H + h];
      w_b0 = reinterpret_cast<const uint32_t *>(gb)[(rowbase + ts) * p.H + h];
      w_a1 = reinterpret_cast<const uint32_t *>(ga)[(rowbase + tn) * p.H + h];
      w_b1 = reinterpret_cast<const uint32_t *>(gb)[(rowbase + tn) * p.H + h];
    }
  } else {
    constexpr int NY = 2 * RM * SPW * 2 / 16, NL = 2 * RM * kAR * 4 / 16;
    static_assert(offsetof(SM, w1) == offsetof(SM, y) + RM * SPW * 2, "Y and W1 adjacent");
    static_assert(offsetof(SM, mc) == offsetof(SM, lc) + RM * kAR * 4, "lc and mc adjacent");
    constexpr int NC = kTreeWaves - 1;
#pragma unroll
    for (int x = 0; x < (NY + 64 * NC - 1) / (64 * NC); ++x) {
      const int i = (tw - 1) * 64 + lane + 64 * NC * x;
      if (i < NY) reinterpret_cast<uint4 *>(s.y)[i] = make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int x = 0; x < (NL + 64 * NC - 1) / (64 * NC); ++x) {
      const int i = (tw - 1) * 64 + lane + 64 * NC * x;
      if (i < NL) reinterpret_cast<uint4 *>(s.lc)[i] = make_uint4(0u, 0u, 0u, 0u);
    }
    // q and k rows straight into LDS, 1 KiB chunks dealt over tw 1..3: each wave instruction
    // fills 64 consecutive 16-byte chunks; lane l of chunk qi holds physical chunk 64 qi + l
    // and fetches the logical chunk that the swizzle places there.  Rows past the node count
    // fetch row n-1 (never used).
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(static_cast<const T *>(p.q) + (rowbase * p.H + h) * (size_t)D), 0, nb, 0x00020000);
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(static_cast<const T *>(p.k) + (rowbase * p.H + h) * (size_t)D), 0, nb, 0x00020000);
#pragma unroll
    for (int x = 0; x < (2 * QMAX + NC - 1) / NC; ++x) {
      const int c = (tw - 1) + NC * x;
      if (c < 2 * QMAX) {
        const int qi = c < QMAX ? c : c - QMAX;
        const int pc = 64 * qi + lane, r = pc / CPR, cc = (pc % CPR) ^ (r & (CPR - 1));
        const unsigned off = (unsigned)((min(r, nl) * (int)rstride + cc * CH) * (int)sizeof(T));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(c < QMAX ? rq : rk,
                                                 (lds_void_t *)(s.qk + (c < QMAX ? 0 : SM::ROWB) + 1024 * qi), 16,
                                                 off, 0, 0, 0);
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();  // the counter is clear; the product waves may queue their loads
  // keep every use of tw 0's loaded values (and the wait for them) after the barrier
  asm volatile("" : "+v"(w_mask), "+v"(my_mask), "+v"(w_par), "+v"(w_a0), "+v"(w_b0), "+v"(w_a1), "+v"(w_b1));

  uint32_t ancw[5] = {0u, 0u, 0u, 0u, 0u};  // slot of the ancestor at depth e, byte e
  int d_me = 0;
  if (tw == 0) {
    const auto gate = [](uint32_t x) { return BF16IN ? __uint_as_float(x << 16) : __uint_as_float(x); };
    const float a0 = gate(w_a0), b0 = gate(w_b0), a1 = gate(w_a1), b1 = gate(w_b1);
    if (lane < n) s.mask[lane] = my_mask;
    if constexpr (RM == kMaxSlots) {
      if (lane == 63 && n == kMaxSlots) s.mask[64] = w_mask;  // slot 64 has no lane of its own
    }
    if (lane == 0 && my_mask != 0ull) s.bad = 1;  // the root has no ancestors
    const bool tv = t_me < n;
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
      if (a == t_me) {
        av = a1;
        bv = b1;
      }
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
  tree_sync(&s.sync, &s.bad, kTreeWaves, lane);  // rows, masks, gates and cleared regions are in LDS

  // ---- Gram tiles [Q; K] K^T of the lower node triangle, dealt between the tree waves ----
  // Transposed: lane (g, t) owns node t = 16 mt + l16 and gets k_s . k_t and k_s . q_t for
  // s = 16 nt + 4 g + 0..3.  Entries of ancestor pairs are kept at depth(s) = (t's
  // ancestors-or-self in slots 0..s) - 1 (the k.k ones times b_t, the factor the path solve
  // applies); the rest go to padding entries 17..19.  Rows past the node count read finite
  // or arbitrary LDS contents; the entries they produce are never kept.
#pragma unroll
  for (int mt = 0; mt < NT; ++mt) {
#pragma unroll
    for (int nt = 0; nt <= mt; ++nt) {
      if ((mt * (mt + 1) / 2 + nt) % kTreeWaves != kTreeWaves - 1 - tw || mt >= ntl) continue;
      const int tme = 16 * mt + l16, ra = min(tme, nl);
      const int rb = 16 * nt + l16;
      f32x4 gk4 = {0.f, 0.f, 0.f, 0.f}, gq4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        bf16x8 aqh, aql, akh, akl, bh, bl;
        row_frag<D, BF16IN>(qrow, tme, 32 * ks + 8 * g4, aqh, aql);
        row_frag<D, BF16IN>(krow, tme, 32 * ks + 8 * g4, akh, akl);
        row_frag<D, BF16IN>(krow, rb, 32 * ks + 8 * g4, bh, bl);
        gk4 = mfma_bf16(bh, akh, gk4);
        gq4 = mfma_bf16(bh, aqh, gq4);
        if constexpr (!BF16IN) {
          gk4 = mfma_bf16(bl, akh, gk4);
          gk4 = mfma_bf16(bh, akl, gk4);
          gq4 = mfma_bf16(bl, aqh, gq4);
          gq4 = mfma_bf16(bh, aql, gq4);
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
  tree_sync(&s.sync, &s.bad, 2 * kTreeWaves, lane);  // the compact Gram rows are complete

  // ---- tw 0: path solve, one lane per node, then the node's Y and W1 rows (fp16) --------
  if (tw == 0) {
    const bool tv = t_me < n;
    const int t = tn;
    const int dmax = wave_max_i32(tv ? d_me : 0);
    auto anc_at = [&](int e) -> int { return (int)((ancw[e >> 2] >> (8 * (e & 3))) & 0xffu); };
    float z[kAR];  // right-hand side q_t . k_{anc e}; zero beyond the depth
#pragma unroll
    for (int v = 0; v < kAR / 4; ++v) {
      const float4 x = reinterpret_cast<const float4 *>(&s.mc[t * kAR])[v];
      z[4 * v] = x.x;
      z[4 * v + 1] = x.y;
      z[4 * v + 2] = x.z;
      z[4 * v + 3] = x.w;
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
    if (tv) {
#pragma unroll
      for (int e = 0; e <= kMaxP; ++e) {
        if (e <= d_me) {
          const int a = anc_at(e);
          const int pos = t * SPW + w1_pos(a);
          s.w1[pos] = (_Float16)(s.cwl[e][lane] * z[e]);
          s.y[pos] = (_Float16)(s.beta[a] * z[e]);
        }
      }
    }
  } else if (tw == 1 && lane == 0) {
    // the root: Y[0, 0] = W1[0, 0] = b_0 (q_0 . k_0)
    const _Float16 w = (_Float16)(s.beta[0] * s.mc[0]);
    s.w1[0] = w;
    s.y[0] = w;
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): Y and W1 are written
  __builtin_amdgcn_s_barrier();        // (1) the product waves may form V^T W1^T

  // ---- E = g (Q - Y K) on MFMA, channel tiles dealt over the tree waves, written as fp16
  //      over the q rows --------------------------------------------------------------------
  // Per channel tile ct: K^T in the C layout (lane (g, c): nodes 4 g + 0..3 of each 16-node
  // tile at channel 16 ct + c) through products with the negated identity (exact), packed as
  // the A operand; then E^T tile by node tile with Q^T as the initial C tile and Y^T as the
  // B operand (Y is zero above the diagonal).  Lane (g, t) ends with E[t][16 ct + 4 g + 0..3].
  static_assert(NW % kTreeWaves == 0, "channel tiles dealt evenly");
  // Straight-line code over all node tiles (rows past the node count are clamped, their K
  // entries zeroed and their E rows never used), so the LDS reads of a channel tile can all
  // be issued ahead of its products.
#pragma unroll
  for (int cc = 0; cc < NW / kTreeWaves; ++cc) {
    const int ct = tw + kTreeWaves * cc;
    f16x8 kt[KSS];
#pragma unroll
    for (int mt = 0; mt < 2 * KSS; ++mt) {
      f32x4 c = {0.f, 0.f, 0.f, 0.f};
      if constexpr (true) {
        if (mt < NT) {
          const int r = min(16 * mt + l16, nl);
          if constexpr (BF16IN) {
            s16x4 nid;  // bf16 -1 on the diagonal
#pragma unroll
            for (int e = 0; e < 4; ++e) nid[e] = (short)((4 * g4 + e == l16) ? 0xbf80 : 0);
            const s16x4 a = *reinterpret_cast<const s16x4 *>(krow + swz<D, 8>(r, 16 * ct + 4 * g4));
            c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, nid, c, 0, 0, 0);
          } else {
            f16x4 nid, a;
            const f32x4 kv = row4<D, false>(krow, r, 16 * ct + 4 * g4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              nid[e] = (_Float16)((4 * g4 + e == l16) ? -1.f : 0.f);
              a[e] = (_Float16)kv[e];
            }
            c = mfma16_f16(a, nid, c);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) c[i] = (16 * mt + 4 * g4 + i < n) ? c[i] : 0.f;
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) kt[mt >> 1][4 * (mt & 1) + i] = (_Float16)c[i];
    }
    // Scheduling fences: this channel tile's K^T fragments are packed before its products,
    // and the next tile's only after this tile's E rows (which read the last products'
    // results).  An interleaved schedule, in which VALU packing of the next tile's fragments
    // rewrote the B operand registers of an MFMA still waiting on the previous MFMA's
    // accumulator, gave wrong E entries in workgroups sharing a CU.
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int mt = 0; mt < NT; ++mt) {
      const int t = 16 * mt + l16;
      const int tq = min(t, nl);
      f32x4 acc = row4<D, BF16IN>(qrow, tq, 16 * ct + 4 * g4);
#pragma unroll
      for (int kk = 0; kk < KSS; ++kk) {
        if (32 * kk > 16 * mt + 15) break;
        acc = mfma_f16(kt[kk], hfrag(s.y + tq * SPW + 32 * kk + 8 * g4), acc);
      }
      const float gt = s.gamma[t];
      f16x4 ev;
#pragma unroll
      for (int i = 0; i < 4; ++i) ev[i] = (_Float16)(gt * acc[i]);
      // rows n..RM-1 are unused scratch; rows past RM do not exist
      if (mt < NT - 1 || t < RM) *reinterpret_cast<f16x4 *>(erow + swz<D, 8>(t, 16 * ct + 4 * g4)) = ev;
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): E is written
  __builtin_amdgcn_s_barrier();        // (2) the product waves may read E
  __builtin_amdgcn_s_barrier();        // (3) every output row is staged
  store_rows<D>(p, ostage, n, rowbase, h, 64 * wave + lane, 64 * (NW + kTreeWaves));
}

template <int D, bool BF16IN, int NT>
hipError_t launch_one(const VerifyParams &p, hipStream_t stream) {
  const unsigned units = (unsigned)(p.L * p.B * p.H);
  hipLaunchKernelGGL((verify_kernel<D, BF16IN, NT>), dim3(units), dim3(VerifyShape<D, BF16IN, NT>::NTH), 0,
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
