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
// root..t.  Unrolling the recurrence along t's path gives S_t = g_t S0 + sum_s (g_t/g_s) b_s
// k_s w_s^T over the ancestors-or-self s of t, with pseudo-values w that solve a system
// triangular along root paths.  Collecting the coefficients of each row: for node t with
// ancestors-or-self anc e at depths e = 0..d_t, let z solve (deepest first)
//     z[e] + sum_{e2 > e} z[e2] b_{anc e2} (k_{anc e2} . k_{anc e}) = q_t . k_{anc e};
// with Y[t, e] = b_{anc e} z[e] and W1[t, e] = (g_t / g_{anc e}) Y[t, e],
//     o_t = g_t (S0^T q_t - sum_e Y[t, e] S0^T k_{anc e}) + sum_e W1[t, e] v_{anc e}
//         = g_t S0^T q_t + sum_e W1[t, e] U[anc e],     U[s] = v_s - g_s S0^T k_s.
// So the committed state S0 (d_k x d_v fp32), the only large operand, enters through the
// dense products A_q = Q S0 and A_k = K S0 over the rows as they are, which need neither
// the tree nor the gates; the tree enters through small work on q, k, a, b only (Gram
// entries of ancestor pairs, one path solve per node), and the two meet in one product of
// the (sparse, lower triangular) W1 rows with U.
//
// Precision.  The products A_q and A_k are fp32-exact: each fp32 state entry is split into
// three bf16 parts hi + mid + lo that hold its 24-bit significand exactly (hi = RN(x),
// mid = RN(x - hi), lo = x - hi - mid, every difference exact in fp32), and every part
// multiplies the bf16 rows exactly on MFMA with fp32 accumulation.  fp32 rows are split the
// same way (six of the nine part products; the three dropped ones are below 2^-24 of the
// term), and so are W1 and U in their product.  The Gram entries are exact products
// accumulated in fp32 (split likewise for fp32 rows), and the path solves and gates run in
// fp32.
//
// Work decomposition: one workgroup per (layer, request, head), two resident per CU, with two
// kinds of waves.
//  * d/16 product waves, wave w owning value channels [16 w, 16 w + 16): they stream the q,
//    k and v rows into LDS (buffer loads to LDS), gather this head's state columns from the
//    [d_k][d_v] layout (lane (g, c) holds S0[32 ks + 8 g + e][16 w + c], an operand of a
//    16x16x32 product), split them as they land, and form A_k and A_q for their channels with
//    the row tiles read from LDS; then the W1 U product and the output rows.
//  * four tree waves: wave 0 loads the per-node inputs and does the per-node prologue; waves
//    1..3 clear the compact Gram rows.  Together they compute the Gram tiles [Q; K] K^T of the
//    lower node triangle, then wave 0 does the per-node path solves (one lane per node), and
//    all four form the W1 rows as dense bf16 parts, which they write over the q and k rows
//    once those are dead: the operand of the W1 U product.
// Rows 0..63 go through 16-row MFMA tiles; a 65th row (a tree of 64 drafts) rides in one
// extra tile of its own, and its W1 row is summed on VALU.
//
// With the previous step's commit first (CM), the same workgroup first recomputes the state of
// the previous step's accepted node (same page, Prerequisites > speculative decoding and >
// hybrid recurrent architecture: greedy acceptance, then the accepted path's state): tree wave
// 0 walks the previous tree's acceptance, the product waves hold their whole state slice in
// registers, fetch the accepted path's k and v rows into LDS, apply the path's rows in order
// (S <- a S + k (b (v - a k . S))^T, fp32), write the slice back in place and go on to the
// products with it.  The state is then read once and written once per step.
//
// MFMA operand registers are refilled only after the products that read them have completed:
// every chain of products is fenced off from the code that refills its operands, and before a
// wave overwrites registers that earlier products read, it reads each accumulator those
// products wrote (a VALU read of an MFMA result, which the compiler delays by the required
// wait states, so the products have finished).

#include <type_traits>

#include "commit_device.h"
#include "gdntree_internal.h"

namespace gdntree {
namespace {

constexpr int kAR = 20;  // compact coefficient row: depths 0..16, padded to five 16-byte vectors
constexpr int kLdsBytes = 160 * 1024;
constexpr int kTreeWaves = 4;

template <bool BF16IN>
struct InT;
template <>
struct InT<true> { typedef uint16_t T; };
template <>
struct InT<false> { typedef float T; };

// NT 16-row tiles of rows (rows 0 .. 16 NT - 1) plus, with X65, the 65th row.
template <int D, bool BF16IN, int NT, bool X65>
struct VerifyGeom {
  typedef typename InT<BF16IN>::T T;
  static constexpr int RM = 16 * NT + (X65 ? 1 : 0);                       // rows held
  static constexpr int ROWB = (RM * D * (int)sizeof(T) + 1023) / 1024 * 1024;  // whole 1 KiB loads
  static constexpr int NB = (NT + 1) / 2;  // 32-slot blocks of the W1 U product
  static constexpr int SPD = 32 * NB;      // slots per dense W1 row
  static constexpr int PR = 16 * NT;       // dense W1 rows (the 65th row is kept apart, in fp32)
  static constexpr int CPW = SPD / 8;      // 16-byte chunks per dense W1 row
  static constexpr bool PL_R0 = 3 * PR * SPD * 2 <= 2 * ROWB;  // the dense parts fit over q and k
  static constexpr int NPW = D / 16;       // product waves
  static constexpr int WAVES = NPW + kTreeWaves;
  static constexpr int NTH = 64 * WAVES;
};

template <int D, bool BF16IN, int NT, bool X65, bool CM>
struct VerifySmem {
  typedef VerifyGeom<D, BF16IN, NT, X65> G;
  typedef typename G::T T;
  // q rows | k rows; once they are dead, the dense W1 rows as three bf16 parts (when they fit):
  // W1[t][s] for t < PR, s < SPD, zero off t's ancestors-or-self.  Within a 32-slot block,
  // slot 16 h + 4 g + i sits at 8 g + 4 h + i, so that one lane's operand fragment is one
  // 16-byte chunk; chunks are XOR-swizzled by the row, so that 16 consecutive rows read at one
  // chunk hit distinct banks.  Output rows wider than the inputs are staged here at the end.
  alignas(16) unsigned char r0[2 * G::ROWB];
  alignas(16) unsigned char r1[G::ROWB];   // v rows; then the output rows (when they fit)
  alignas(16) uint16_t plx[G::PL_R0 ? 8 : 3 * G::PR * G::SPD];  // the dense W1 parts otherwise
  alignas(16) float cy[G::RM * kAR];       // Gram b_t k_t.k_s (strict ancestors s)
  alignas(16) float cw[G::RM * kAR];       // Gram q_t.k_s (ancestors-or-self s), then W1[t, e] (compact)
  alignas(16) float w64[X65 ? 64 : 4];     // W1[64][s], s < 64, in fp32
  alignas(16) unsigned long long mask[G::RM];
  float gamma[G::RM];                      // path gate g_t
  float beta[G::RM];                       // b per node
  float cwl[kMaxAnc][64];                  // W1 weights b_{anc e} g_t / g_{anc e}, per depth and lane
  int bad;
  int sync;                                // tree-wave phase counter
  // The previous step's commit: its accepted path's k rows (rows 0..16) and v rows (rows
  // 17..33), the path's slots, the previous tree's tokens, tau, the bonus token, and a counter
  // of the product waves whose path rows have landed.
  alignas(16) unsigned char cpath[CM ? 2 * kMaxAnc * D * (int)sizeof(T) : 16];
  int cslot[kMaxAnc];
  int ctok[CM ? kMaxSlots : 1];
  int ctau, cbonus, csync;
};

template <int D, bool BF16IN, int NT, bool X65, bool CM>
struct VerifyShape {
  typedef VerifyGeom<D, BF16IN, NT, X65> G;
  static constexpr int LDS = (int)sizeof(VerifySmem<D, BF16IN, NT, X65, CM>);
  static_assert(LDS <= kLdsBytes, "a workgroup's LDS fits a CU");
  static constexpr int WG_PER_CU = kLdsBytes / LDS < 2 ? 1 : 2;
  // A workgroup's waves are dealt over the CU's four SIMDs, so the register budget must let
  // every SIMD hold ceil(WAVES / 4) waves of each resident workgroup.
  static constexpr int WPEU = WG_PER_CU * ((G::WAVES + 3) / 4);
};

// Rows live in LDS unpadded with their 16-byte chunks XOR-swizzled by the row index, so that
// 16 consecutive rows read at one logical column hit distinct banks.
template <int D, int CH>
__device__ __forceinline__ int swz(int r, int i) {
  constexpr int CPR = D / CH;
  return r * D + (((i / CH) ^ (r & (CPR - 1))) * CH) + (i % CH);
}

typedef __attribute__((address_space(3))) void lds_void_t;

// Workgroup barrier that is also a compiler barrier for memory operations: the s_barrier
// builtin alone does not order memory accesses at the IR level, so loads of LDS data that
// other waves write before the barrier could otherwise be moved above it.
__device__ __forceinline__ void wg_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

__device__ __forceinline__ bf16x8 frag16(const void *p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(p));
}

// x = hi + mid + lo exactly, each part bf16 (round to nearest even): x - hi and x - hi - mid
// are exact in fp32 and the last difference fits bf16's significand.  Two elements at a time,
// one packed conversion per part.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void split3(const float *x, bf16x8 &hi, bf16x8 &mid, bf16x8 &lo) {
#pragma unroll
  for (int i = 0; i < 8; i += 2) {
    const f32x2 v = {x[i], x[i + 1]};
    const bf16x2 h = __builtin_convertvector(v, bf16x2);
    const f32x2 r = v - __builtin_convertvector(h, f32x2);
    const bf16x2 m = __builtin_convertvector(r, bf16x2);
    const bf16x2 l = __builtin_convertvector(r - __builtin_convertvector(m, f32x2), bf16x2);
    hi[i] = h[0]; hi[i + 1] = h[1];
    mid[i] = m[0]; mid[i + 1] = m[1];
    lo[i] = l[0]; lo[i + 1] = l[1];
  }
}

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Product of a bf16 operand (exact) with an exactly split fp32 operand (three parts), the
// split operand second (B) or first (A).
__device__ __forceinline__ f32x4 mfma_x3(bf16x8 a, const bf16x8 &bh, const bf16x8 &bm, const bf16x8 &bl, f32x4 c) {
  c = mfma_bf16(a, bl, c);
  c = mfma_bf16(a, bm, c);
  return mfma_bf16(a, bh, c);
}
__device__ __forceinline__ f32x4 mfma_x3t(const bf16x8 &ah, const bf16x8 &am, const bf16x8 &al, bf16x8 b, f32x4 c) {
  c = mfma_bf16(al, b, c);
  c = mfma_bf16(am, b, c);
  return mfma_bf16(ah, b, c);
}
// Product of two exactly split fp32 operands: the six part products down to 2^-16 relative.
__device__ __forceinline__ f32x4 mfma_x6(const bf16x8 &ah, const bf16x8 &am, const bf16x8 &al, const bf16x8 &bh,
                                         const bf16x8 &bm, const bf16x8 &bl, f32x4 c) {
  c = mfma_bf16(ah, bl, c);
  c = mfma_bf16(am, bm, c);
  c = mfma_bf16(al, bh, c);
  c = mfma_bf16(ah, bm, c);
  c = mfma_bf16(am, bh, c);
  return mfma_bf16(ah, bh, c);
}

// Eight consecutive elements of one LDS row (a 16-byte chunk for bf16, two for fp32), as the
// operand fragment of a product that contracts over d: the bf16 row itself, or an fp32 row
// split in three.
template <int D, bool BF16IN>
__device__ __forceinline__ void row_frag(const typename InT<BF16IN>::T *rows, int r, int col, bf16x8 &hi,
                                         bf16x8 &mid, bf16x8 &lo) {
  if constexpr (BF16IN) {
    hi = frag16(rows + swz<D, 8>(r, col));
  } else {
    const float4 a = *reinterpret_cast<const float4 *>(rows + swz<D, 4>(r, col));
    const float4 b = *reinterpret_cast<const float4 *>(rows + swz<D, 4>(r, col + 4));
    const float f[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    split3(f, hi, mid, lo);
  }
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

__device__ __forceinline__ int imin(int a, int b) { return a < b ? a : b; }

__device__ __forceinline__ float bperm_f32(int lane_src, float x) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(lane_src << 2, __float_as_int(x)));
}
__device__ __forceinline__ float to_f32(uint16_t x) { return bf16_bits_to_f32(x); }
__device__ __forceinline__ float to_f32(float x) { return x; }

// Reads accumulator element 0 with a VALU instruction and keeps the value alive, so that the
// products that wrote it have completed before anything after this point issues.
__device__ __forceinline__ void drain(const f32x4 &acc) {
  const int s = __builtin_amdgcn_readfirstlane(__float_as_int(acc[0]));
  asm volatile("" ::"s"(s));
}

// The tree waves meet here: each finishes its own memory work (loads into LDS included),
// counts itself in, and waits for the others.  The wait is bounded; a wave that gives up marks
// the request bad (NaN outputs) instead of hanging.
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

template <int D, bool BF16IN, int NT, bool X65, bool CM>
__global__ __launch_bounds__((VerifyGeom<D, BF16IN, NT, X65>::NTH), (VerifyShape<D, BF16IN, NT, X65, CM>::WPEU))
void verify_kernel(VerifyParams p) {
  typedef VerifyGeom<D, BF16IN, NT, X65> G;
  typedef VerifySmem<D, BF16IN, NT, X65, CM> SM;
  typedef typename G::T T;
  constexpr int RM = G::RM, ROWB = G::ROWB, NTH = G::NTH;
  constexpr int CH = 16 / (int)sizeof(T), CPR = D / CH;
  constexpr int KS = D / 32;               // MFMA k-steps over d_k
  constexpr int NPW = G::NPW;              // product waves
  constexpr int QMAX = ROWB / 1024;        // 1 KiB row chunks per matrix
  constexpr int NTG = NT + (X65 ? 1 : 0);  // Gram node tiles (the 65th row has one of its own)
  constexpr int SPD = G::SPD, CPW = G::CPW;
  constexpr int NC = kTreeWaves - 1;       // tree waves that load rows
  static_assert(2 * ROWB >= RM * D * 4, "fp32 output rows fit over the q and k rows");
  __shared__ SM s;

  const int tid = threadIdx.x, lane = tid & 63, g4 = lane >> 4, l16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int u = blockIdx.x;  // (layer, request, head)
  const int h = u % p.H, lb = u / p.H, b = lb % p.B;
  // n_nodes is read-only here: a scalar load.  The row and per-node loads do not wait for it:
  // they cover all R slots of the request (slots past the node count are read, never used).
  const int32_t __attribute__((address_space(4))) *nn_c =
      (const int32_t __attribute__((address_space(4))) *)p.n_nodes;
  const int n = nn_c[b];
  const bool valid = n >= 1 && n <= p.R;  // no output for a request with an impossible node count
  const int nl = n - 1, rl = p.R - 1;
  const int ntl = (imin(n, 16 * NT) + 15) / 16;  // MFMA row tiles in use
  const bool row64 = X65 && n == 65;             // the 65th row
  const size_t rowbase = (size_t)lb * p.R;
  const size_t rstride = (size_t)p.H * D;  // elements between consecutive slots of one head
  const T *qrow = reinterpret_cast<const T *>(s.r0);
  const T *krow = reinterpret_cast<const T *>(s.r0 + ROWB);
  const T *vrow = reinterpret_cast<const T *>(s.r1);
  uint16_t *pl = G::PL_R0 ? reinterpret_cast<uint16_t *>(s.r0) : s.plx;  // dense W1 part 0; parts 1, 2 follow
  // Output rows are staged over the v rows when they fit there, else over the q and k rows once
  // the dense W1 parts are read.
  const bool stage_v = (p.out_bf16 ? 2 : 4) <= (int)sizeof(T);
  unsigned char *stg = stage_v ? s.r1 : s.r0;

  // ---- the dense W1 rows as three bf16 parts: item (t, mb, g) is row t's slots
  // 32 mb + 16 h + 4 g + i, one 16-byte chunk per part; W1[t][s] is the compact entry at s's
  // depth on t's path, or zero.  The tree waves compute their items once the compact rows are
  // solved and write them over the q and k rows once those are dead.
  constexpr int IPR = G::NB * 4;                       // items per row
  constexpr int PIT = G::PR * IPR;                     // items
  constexpr int PXN = (PIT + 64 * kTreeWaves - 1) / (64 * kTreeWaves);  // per tree lane
  auto fill_item = [&](int it, bf16x8 &xh, bf16x8 &xm, bf16x8 &xl) {
    const int t = it / IPR, mb = (it % IPR) >> 2, g = it & 3;
    const unsigned long long aset = t < n ? ((s.mask[t] << 1) | 1ull) : 0ull;
    // the block's 32 slot flags, and t's ancestors-or-self in the blocks below it
    const uint32_t wb = (uint32_t)(aset >> (32 * mb));
    const int below = mb ? __popc((uint32_t)aset) : 0;
    float xv[8];
    // (each entry read unconditionally, at a clamped index, then selected, so that the eight
    // reads are in flight together rather than one conditional read and wait each)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int q = 16 * (e >> 2) + 4 * g + (e & 3);            // slot 32 mb + q
      const int d = below + __popc(wb & ((2u << q) - 1u)) - 1;  // its depth on t's path
      const float x = s.cw[imin(t, RM - 1) * kAR + imin(max(d, 0), kAR - 1)];
      xv[e] = ((wb >> q) & 1u) ? x : 0.f;
    }
    split3(xv, xh, xm, xl);
  };
  auto fill_off = [&](int it) {
    const int t = it / IPR, mb = (it % IPR) >> 2, g = it & 3;
    return t * SPD + 8 * ((4 * mb + g) ^ (t & (CPW - 1)));
  };

  // ---- the staged rows to HBM by every wave: whole rows, 16-byte pieces, consecutive lanes
  // along a row; a fixed number of pieces per lane, the ones past the rows in use falling
  // outside the buffer range (the hardware drops them) -------------------------------------
  auto store_rows = [&]() {
    const int oes = p.out_bf16 ? 2 : 4;
    const int lcpr = p.out_bf16 ? (D == 128 ? 4 : 3) : (D == 128 ? 5 : 4);  // log2 chunks per row
    const int cpr = 1 << lcpr;
    const unsigned ostride = (unsigned)(p.H * D * oes);
    char *obase = static_cast<char *>(p.o) + (rowbase * p.H + h) * (size_t)D * oes;
    const int orange = ((n - 1) * p.H * D + D) * oes;
    const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(obase, 0, orange, 0x00020000);
    constexpr int PIECES = (RM * D * 4 / 16 + NTH - 1) / NTH;  // enough for fp32 rows
    const int nch = n * cpr;
#pragma unroll
    for (int x = 0; x < PIECES; ++x) {
      const int c = tid + NTH * x;
      const int r = imin(c >> lcpr, RM - 1), lc = c & (cpr - 1);
      const u32x4 v = *reinterpret_cast<const u32x4 *>(stg + 16 * (r * cpr + (lc ^ (r & (cpr - 1)))));
      const int off = c < nch ? (int)((unsigned)r * ostride + 16u * lc) : orange;
      __builtin_amdgcn_raw_buffer_store_b128(v, ro, off, 0, 0);
    }
  };

  if (wave < NPW) {
    // ================================ product waves ==================================
    // q, k and v rows straight into LDS, 1 KiB chunks dealt over the product waves (which
    // write no LDS before these have landed): each wave instruction fills 64 consecutive
    // 16-byte chunks; lane l of chunk qi holds physical chunk 64 qi + l and fetches the logical
    // chunk that the swizzle places there.  Rows past the slot count fetch slot R-1 (never
    // used).  They are queued ahead of the state loads below.
    {
      const size_t hoff = (rowbase * p.H + h) * (size_t)D;
      const int nb = (int)((rl * rstride + D) * sizeof(T));  // byte range of this head's slots
      const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
          (void *)(static_cast<const T *>(p.q) + hoff), 0, nb, 0x00020000);
      const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
          (void *)(static_cast<const T *>(p.k) + hoff), 0, nb, 0x00020000);
      const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
          (void *)(static_cast<const T *>(p.v) + hoff), 0, nb, 0x00020000);
#pragma unroll
      for (int x = 0; x < (3 * QMAX + NPW - 1) / NPW; ++x) {
        const int c = wave + NPW * x;
        if (c < 3 * QMAX) {
          const int mat = c / QMAX, qi = c % QMAX;
          const int pc = 64 * qi + lane, r = pc / CPR, cc = (pc % CPR) ^ (r & (CPR - 1));
          const unsigned off = (unsigned)((imin(r, rl) * (int)rstride + cc * CH) * (int)sizeof(T));
          unsigned char *dst = (mat == 2 ? s.r1 : s.r0 + mat * ROWB) + 1024 * qi;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(mat == 0 ? rq : (mat == 1 ? rk : rv), (lds_void_t *)dst, 16,
                                                   off, 0, 0, 0);
        }
      }
    }
    wg_barrier();  // (0)
    if (!CM && !valid) {  // (with a commit, the commit is done first)
      __builtin_amdgcn_s_waitcnt(0);  // loads into this workgroup's LDS land before it ends
      return;
    }
    const int j = 16 * wave + l16;  // this lane's value channel (K pass and the 65th row)
    // State fragments in the [d_k][d_v] layout: lane (g, c) gathers S0[32 ks + 8 g + e][j],
    // 16 consecutive channels (64 bytes) per row and instruction.  The fragment of the next
    // k-step (two with at most three row tiles, where the registers allow it) is in flight while
    // the current one is split and multiplied (register budget of two resident workgroups per
    // CU).  With a commit first, the wave holds all its fragments (the previous committed
    // state), updates them, writes them back and multiplies them as they are.
    constexpr int KW = NT <= 3 ? 2 : 1;
    constexpr int KG = CM ? KS : KW;  // fragments gathered before barrier (1)
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(p.state) + (size_t)u * D * D, 0, D * D * 4, 0x00020000);
    const int voff = (8 * g4 * D + j) * 4;
    float raw[KS][8];
    auto gather = [&](int ks) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        raw[ks][e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, voff, (32 * ks + e) * D * 4, 0));
    };
#pragma unroll
    for (int ks = 0; ks < KG; ++ks) gather(ks);
    // vmcnt(8 KG): this wave's row loads have landed (loads complete in order; the state loads
    // just issued may still be in flight)
    static_assert(8 * KG < 64, "the wait count fits");
    __builtin_amdgcn_s_waitcnt(((8 * KG) & 15) | ((8 * KG) >> 4 << 14) | (7 << 4) | (15 << 8));
    wg_barrier();  // (1) the q, k, v rows and the per-node data are in LDS (and the accepted path)

    if constexpr (CM) {
      // ---- the previous step's commit along its accepted path (tau rows, root first): for
      // each row, S <- a (S - b k (k . S)) + b k v^T = a S + k (b (v - a k . S))^T, in fp32, on
      // this wave's fragments; the path's k and v rows are fetched into LDS by the product
      // waves together, the gates into registers (lane x: path row x) ----------------------
      const int tau = __builtin_amdgcn_readfirstlane(s.ctau);
      if (tau > 0) {
        constexpr int RB = D * (int)sizeof(T), CPRW = RB / 16;
        constexpr int PROUNDS = (kMaxAnc * CPRW + 64 * NPW - 1) / (64 * NPW);
        const size_t pvoff = ((size_t)lb * p.pv_R * p.H + h) * D;
        const int pnb = (int)(((p.pv_R - 1) * rstride + D) * sizeof(T));
        const __amdgpu_buffer_rsrc_t pk = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(static_cast<const T *>(p.pv_k) + pvoff), 0, pnb, 0x00020000);
        const __amdgpu_buffer_rsrc_t pv = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(static_cast<const T *>(p.pv_v) + pvoff), 0, pnb, 0x00020000);
#pragma unroll
        for (int x = 0; x < PROUNDS; ++x) {
          const int c = 64 * (wave + NPW * x) + lane;  // 16-byte chunk c of the path's rows
          if (c < tau * CPRW) {
            const int r = c / CPRW, cc = c - r * CPRW;
            const unsigned off = (unsigned)((s.cslot[r] * (int)rstride + cc * CH) * (int)sizeof(T));
            __builtin_amdgcn_raw_ptr_buffer_load_lds(pk, (lds_void_t *)(s.cpath + 1024 * (wave + NPW * x)), 16, off,
                                                     0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                pv, (lds_void_t *)(s.cpath + kMaxAnc * RB + 1024 * (wave + NPW * x)), 16, off, 0, 0, 0);
          }
        }
        float pa = 0.f, pb = 0.f;
        if (lane < tau) {
          const size_t gi = ((size_t)lb * p.pv_R + s.cslot[lane]) * p.H + h;
          pa = load_elem(static_cast<const T *>(p.pv_alpha), gi);
          pb = load_elem(static_cast<const T *>(p.pv_beta), gi);
        }
        __builtin_amdgcn_s_waitcnt(0);  // the state fragments, path rows and gates have landed
        if (lane == 0) __hip_atomic_fetch_add(&s.csync, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        int spins = 0;
        bool met = true;
        while (__hip_atomic_load(&s.csync, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < NPW) {
          __builtin_amdgcn_s_sleep(1);
          if (++spins > (1 << 22)) {
            met = false;
            break;
          }
        }
        if (!met) {
          s.bad = 1;  // the state stays as it was; the outputs of this unit are NaN
        } else {
          const unsigned char *kb = s.cpath;
          const T *vb = reinterpret_cast<const T *>(s.cpath + kMaxAnc * RB);
          auto kfrag = [&](int r, int ks, float (&kv)[8]) {
            if constexpr (BF16IN) {
              const uint4 x = *reinterpret_cast<const uint4 *>(kb + r * RB + (32 * ks + 8 * g4) * 2);
              const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                kv[2 * i] = __uint_as_float(w[i] << 16);
                kv[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
              }
            } else {
              const float4 x0 = *reinterpret_cast<const float4 *>(kb + r * RB + (32 * ks + 8 * g4) * 4);
              const float4 x1 = *reinterpret_cast<const float4 *>(kb + r * RB + (32 * ks + 8 * g4 + 4) * 4);
              kv[0] = x0.x; kv[1] = x0.y; kv[2] = x0.z; kv[3] = x0.w;
              kv[4] = x1.x; kv[5] = x1.y; kv[6] = x1.z; kv[7] = x1.w;
            }
          };
          for (int r = 0; r < tau; ++r) {
            const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pa), r));
            const float bb = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pb), r));
            float dot4[4] = {0.f, 0.f, 0.f, 0.f};  // k . S over this lane's key rows, one sum per k-step
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
              float kv[8];
              kfrag(r, ks, kv);
#pragma unroll
              for (int e = 0; e < 8; ++e) dot4[ks & 3] = fmaf(kv[e], raw[ks][e], dot4[ks & 3]);
            }
            float dot = (dot4[0] + dot4[1]) + (dot4[2] + dot4[3]);
            dot += __shfl_xor(dot, 16);  // the four lanes of channel j hold its 4 x 32 key rows
            dot += __shfl_xor(dot, 32);
            const float coef = bb * (to_f32(vb[r * D + j]) - a * dot);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {  // k read again rather than held across the exchange
              float kv[8];
              kfrag(r, ks, kv);
#pragma unroll
              for (int e = 0; e < 8; ++e) raw[ks][e] = fmaf(kv[e], coef, a * raw[ks][e]);
            }
          }
          // the committed state, in place
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e)
              __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(raw[ks][e]), rs, voff, (32 * ks + e) * D * 4, 0);
        }
      }
      if (!valid) {
        __builtin_amdgcn_s_waitcnt(0);
        return;
      }
      // the products below take the committed state from these registers (streaming it back
      // from the caches instead measured slower: part of it had left L2 and was read again)
    }

    // The rest of a product wave's work, as straight-line code for each count of row tiles in
    // use (a runtime loop bound over the tiles would keep every accumulator live everywhere).
    auto product_phase = [&](auto ntu_c) {
      constexpr int NTU = decltype(ntu_c)::value;
      constexpr bool R65 = X65 && NTU == NT;  // only a full set of tiles can have a 65th row
      const bool r64 = R65 && row64;
      // ak[mt]: A_k rows 16 mt + 4 g + r, channel j (lane (g, c) = (g, j - 16 w)).
      // aq[mt]: A_q transposed, lane (g, c) holding node 16 mt + c, channels 16 w + 4 g + r.
      f32x4 ak[NTU], aq[NTU];
#pragma unroll
      for (int mt = 0; mt < NTU; ++mt) {
        ak[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        aq[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      // The 65th row's products: one more tile whose row 0 is k_64 and row 1 is q_64 (the other
      // rows repeat q_64 and are never used), so lane (0, c) ends with A_k[64][j] in element 0
      // and A_q[64][j] in element 1.
      f32x4 a65 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        // The split of this k-step starts only after the previous k-step's drains (volatile asm
        // keeps its order), and the next gather only after the split, so at most two raw
        // fragments and one split are live.
        asm volatile("" : "+v"(raw[ks][0]), "+v"(raw[ks][1]), "+v"(raw[ks][2]), "+v"(raw[ks][3]),
                     "+v"(raw[ks][4]), "+v"(raw[ks][5]), "+v"(raw[ks][6]), "+v"(raw[ks][7]));
        bf16x8 sh, sm, sl;
        split3(raw[ks], sh, sm, sl);
        asm volatile("" : "+v"(sh), "+v"(sm), "+v"(sl)::"memory");
        if (!CM && ks + KW < KS) gather(ks + KW);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int mt = 0; mt < NTU; ++mt) {
          bf16x8 xh, xm, xl;
          row_frag<D, BF16IN>(krow, 16 * mt + l16, 32 * ks + 8 * g4, xh, xm, xl);
          if constexpr (BF16IN) ak[mt] = mfma_x3(xh, sh, sm, sl, ak[mt]);
          else ak[mt] = mfma_x6(xh, xm, xl, sh, sm, sl, ak[mt]);
          if constexpr (!BF16IN) drain(ak[mt]);  // fp32 row fragments are split on VALU
          row_frag<D, BF16IN>(qrow, 16 * mt + l16, 32 * ks + 8 * g4, xh, xm, xl);
          if constexpr (BF16IN) aq[mt] = mfma_x3t(sh, sm, sl, xh, aq[mt]);
          else aq[mt] = mfma_x6(sh, sm, sl, xh, xm, xl, aq[mt]);
          if constexpr (!BF16IN) drain(aq[mt]);
        }
        if constexpr (R65) {
          bf16x8 xh, xm, xl;
          row_frag<D, BF16IN>(l16 == 0 ? krow : qrow, 64, 32 * ks + 8 * g4, xh, xm, xl);
          if constexpr (BF16IN) a65 = mfma_x3(xh, sh, sm, sl, a65);
          else a65 = mfma_x6(xh, xm, xl, sh, sm, sl, a65);
          drain(a65);
        }
        // the products of this k-step have completed before the next split overwrites sh, sm, sl
#pragma unroll
        for (int mt = 0; mt < NTU; ++mt) {
          drain(ak[mt]);
          drain(aq[mt]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // From here to the stores this wave is on the launch's critical path (the tree waves are
      // done with their chain): it takes precedence over them on its SIMD.
      __builtin_amdgcn_s_setprio(2);
      // ---- o[t] = g_t A_q[t] + sum_s W1[t][s] U[s] on MFMA, U[s] = v[s] - g_s A_k[s] ---------
      // U takes A_k's place in this lane's registers (rows >= n zero) while the tree waves finish
      // the path solves (the gates and the v rows are in LDS since barrier (1)).
      f32x4 oc[NTU];
#pragma unroll
      for (int mt = 0; mt < NTU; ++mt) {
        const float gq = s.gamma[16 * mt + l16];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          oc[mt][r] = gq * aq[mt][r];  // rows >= n are never stored
          const int t = 16 * mt + 4 * g4 + r;
          ak[mt][r] = t < n ? to_f32(vrow[swz<D, CH>(t, j)]) - s.gamma[t] * ak[mt][r] : 0.f;
        }
      }
      // the 65th row: A_k[64] and A_q[64] sit in lanes (0, c) of a65
      float u64 = 0.f;
      if constexpr (R65) {
        if (r64) u64 = to_f32(vrow[swz<D, CH>(64, j)]) - s.gamma[64] * a65[0];
      }
      wg_barrier();  // (2) nobody reads q or k rows any more; the compact W1 rows are solved
      const bool bad = __builtin_amdgcn_readfirstlane(s.bad) != 0;
      wg_barrier();  // (3) the dense W1 rows are ready; nobody reads the v rows any more

      // Transposed, o^T = U^T W1^T: 16x16x32 products over 32-slot blocks, the contraction
      // index k = 8 g + e of lane (g, c) standing for slot s = 32 mb + 16 (e / 4) + 4 g + e % 4.
      // The A operand of lane (g, c) is then its own U rows of tiles 2 mb and 2 mb + 1 (the K
      // pass's layout, rows 4 g + 0..3) split in three, and the B operand, W1[16 mt + c] at
      // those slots, is one 16-byte chunk of each dense part.  The result has A_q's transposed
      // layout.  The 65th row goes on VALU.
      float p64 = 0.f;  // this lane's share of row 64's sum over s < 64
      constexpr int NBU = (NTU + 1) / 2;  // 32-slot blocks in use
#pragma unroll
      for (int mb = 0; mb < NBU; ++mb) {
        bf16x8 uh, um, ul;
        float ua[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
          ua[e] = (2 * mb + (e >> 2) < NTU) ? ak[imin(2 * mb + (e >> 2), NTU - 1)][e & 3] : 0.f;
        split3(ua, uh, um, ul);
        if constexpr (R65) {
          if (r64) {
            const float4 wa = *reinterpret_cast<const float4 *>(&s.w64[32 * mb + 4 * g4]);
            const float4 wb = *reinterpret_cast<const float4 *>(&s.w64[32 * mb + 16 + 4 * g4]);
            p64 = fmaf(wa.x, ua[0], p64); p64 = fmaf(wa.y, ua[1], p64);
            p64 = fmaf(wa.z, ua[2], p64); p64 = fmaf(wa.w, ua[3], p64);
            p64 = fmaf(wb.x, ua[4], p64); p64 = fmaf(wb.y, ua[5], p64);
            p64 = fmaf(wb.z, ua[6], p64); p64 = fmaf(wb.w, ua[7], p64);
          }
        }
#pragma unroll
        for (int mt = 2 * mb; mt < NTU; ++mt) {
          const int t = 16 * mt + l16;
          const int off = t * SPD + 8 * ((4 * mb + g4) ^ (t & (CPW - 1)));
          const bf16x8 wh = frag16(pl + off), wm = frag16(pl + G::PR * SPD + off);
          const bf16x8 wl = frag16(pl + 2 * G::PR * SPD + off);
          __builtin_amdgcn_sched_barrier(0);
          oc[mt] = mfma_x6(uh, um, ul, wh, wm, wl, oc[mt]);
          drain(oc[mt]);  // these products have completed before the next loads overwrite w*
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      float o64 = 0.f;
      if constexpr (R65) {
        if (r64) {  // the four lanes of a channel folded, then row 64's own term
          p64 += __shfl_xor(p64, 16);
          p64 += __shfl_xor(p64, 32);
          const int d64 = imin((int)__popcll(s.mask[64]), kMaxP);
          o64 = s.gamma[64] * a65[1] + p64 + s.cw[64 * kAR + d64] * u64;
        }
      }
      if (bad) {
#pragma unroll
        for (int mt = 0; mt < NTU; ++mt) oc[mt] = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""),
                                                       __builtin_nanf("")};
        o64 = __builtin_nanf("");
      }
      if (!stage_v) wg_barrier();  // (3b) the dense W1 rows are read before the outputs go over them

      // ---- output rows: lane (g, c) holds node 16 mt + c at channels 16 w + 4 g + 0..3, one
      // 8-byte (bf16) or 16-byte (fp32) piece of a row whose 16-byte chunks are swizzled by the row
#pragma unroll
      for (int mt = 0; mt < NTU; ++mt) {
        const int t = 16 * mt + l16;
        if (t < n) {
          if (p.out_bf16) {
            constexpr int OC = D * 2 / 16;
            const int lc = 2 * wave + (g4 >> 1);
            typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
            const bf16x4 o4 = __builtin_convertvector(oc[mt], bf16x4);
            *reinterpret_cast<uint2 *>(stg + 16 * (t * OC + (lc ^ (t & (OC - 1)))) + 8 * (g4 & 1)) =
                __builtin_bit_cast(uint2, o4);
          } else {
            constexpr int OC = D * 4 / 16;
            const int lc = 4 * wave + g4;
            *reinterpret_cast<f32x4 *>(stg + 16 * (t * OC + (lc ^ (t & (OC - 1))))) = oc[mt];
          }
        }
      }
      if (R65 && r64 && g4 == 0) {
        if (p.out_bf16) {
          constexpr int OC = D * 2 / 16;
          *reinterpret_cast<uint16_t *>(stg + 16 * (64 * OC + (j >> 3)) + 2 * (j & 7)) =
              __builtin_bit_cast(uint16_t, (__bf16)o64);
        } else {
          constexpr int OC = D * 4 / 16;
          *reinterpret_cast<float *>(stg + 16 * (64 * OC + (j >> 2)) + 4 * (j & 3)) = o64;
        }
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's output rows are staged
      wg_barrier();                        // (4) every output row is staged
    };
    static_assert(NT >= 1 && NT <= 4, "one to four row tiles");
    if (ntl == NT) product_phase(std::integral_constant<int, NT>{});
    else if (ntl == 1) product_phase(std::integral_constant<int, 1>{});
    else if (ntl == 2) product_phase(std::integral_constant<int, (NT > 2 ? 2 : 1)>{});
    else product_phase(std::integral_constant<int, (NT > 3 ? 3 : 1)>{});
    store_rows();
    return;
  }

  // ================================== tree waves =====================================
  __builtin_amdgcn_s_setprio(3);  // the tree chain runs beside the state passes: it goes first
  const int tw = wave - NPW;  // 0: per-node tree work and the path solves; 1..3: clears
  const size_t tb = (size_t)b * p.R;
  // tw 0 issues the small per-node loads; tw 1..3 clear the compact Gram rows.
  const int t_me = lane + 1;
  const int tn = imin(t_me, rl);
  const int ts = imin(lane, rl);
  unsigned long long w_mask = 0ull, my_mask = 0ull;
  int w_par = 0;
  uint32_t w_a0 = 0u, w_b0 = 0u, w_a1 = 0u, w_b1 = 0u;  // gate bits
  WalkRegs wr{};  // the previous tree, for the acceptance walk before a commit
  if (tw == 0) {
    if (lane == 0) {
      s.sync = 0;
      s.bad = 0;
      if constexpr (CM) s.csync = 0;
    }
    if constexpr (CM) wr = walk_load(p.pv_parent, p.pv_token, p.pv_target, p.pv_n_nodes, p.pv_R, b, lane);
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
    constexpr int NL = RM * kAR * 4 / 16;  // 16-byte pieces of each compact array
#pragma unroll
    for (int x = 0; x < (NL + 64 * NC - 1) / (64 * NC); ++x) {
      const int i = (tw - 1) * 64 + lane + 64 * NC * x;
      if (i < NL) {
        reinterpret_cast<uint4 *>(s.cy)[i] = make_uint4(0u, 0u, 0u, 0u);
        reinterpret_cast<uint4 *>(s.cw)[i] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the counter and the clears are written
  __builtin_amdgcn_sched_barrier(0);
  wg_barrier();  // (0) the product waves may queue their state loads
  // Before a commit, tree wave 0 walks the previous step's acceptance: the accepted slots and
  // tau for the product waves (and, when asked, the acceptance itself, by the layer-0, head-0
  // workgroup of each request).
  auto cm_walk = [&]() {
    asm volatile("" : "+v"(wr.par0), "+v"(wr.tok0), "+v"(wr.tgt0), "+v"(wr.par1), "+v"(wr.tok1), "+v"(wr.tgt1));
    walk_run(wr, p.pv_R, p.pv_P, lane, s.cslot, s.ctok, &s.ctau, &s.cbonus);
    if (p.acc_len && h == 0 && lb < p.B) {
      const int len = s.ctau;
      if (len > 0 && lane <= p.pv_P) {
        const size_t ab = (size_t)b * (p.pv_P + 1);
        if (lane == 0) p.acc_len[b] = len;
        p.acc_node[ab + lane] = lane < len ? s.cslot[lane] : -1;
        p.acc_tok[ab + lane] = lane < len - 1 ? s.ctok[s.cslot[lane + 1]] : (lane == len - 1 ? s.cbonus : -1);
      }
    }
  };
  if (!valid) {
    if constexpr (CM) {  // no verify output, but the commit still happens
      if (tw == 0) cm_walk();
      __builtin_amdgcn_s_waitcnt(0);
      wg_barrier();  // (1)
    }
    __builtin_amdgcn_s_waitcnt(0);  // the per-node loads complete before the wave ends
    return;
  }
  // keep every use of tw 0's loaded values (and the wait for them) after the barrier
  asm volatile("" : "+v"(w_mask), "+v"(my_mask), "+v"(w_par), "+v"(w_a0), "+v"(w_b0), "+v"(w_a1), "+v"(w_b1));

  uint32_t ancw[5] = {0u, 0u, 0u, 0u, 0u};  // slot of the ancestor at depth e, byte e
  int d_me = 0;
  if (tw == 0) {
    const auto gate = [](uint32_t x) { return BF16IN ? __uint_as_float(x << 16) : __uint_as_float(x); };
    const float a0 = gate(w_a0), b0 = gate(w_b0), a1 = gate(w_a1), b1 = gate(w_b1);
    if (lane < n) s.mask[lane] = my_mask;
    if constexpr (X65) {
      if (lane == 63 && n == kMaxSlots) s.mask[64] = w_mask;  // slot 64 has no lane of its own
    }
    if (lane == 0 && my_mask != 0ull) s.bad = 1;  // the root has no ancestors
    const bool tv = t_me < n;
    const unsigned long long m = w_mask;
    d_me = __popcll(m);
    // the parent's mask is the node mask held by lane parent - 1 (the root's mask is zero)
    const int pl_ = imin(max(w_par - 1, 0), 63);
    const uint32_t pm_lo = (uint32_t)__builtin_amdgcn_ds_bpermute(pl_ << 2, (int)(uint32_t)m);
    const uint32_t pm_hi = (uint32_t)__builtin_amdgcn_ds_bpermute(pl_ << 2, (int)(uint32_t)(m >> 32));
    const unsigned long long pm = w_par == 0 ? 0ull : (((unsigned long long)pm_hi << 32) | pm_lo);
    const bool ok = d_me <= kMaxP && w_par >= 0 && w_par < t_me && m == (pm | (1ull << (t_me - 1)));
    if (tv && !ok) s.bad = 1;
    d_me = imin(d_me, kMaxP);
    float bet[kMaxAnc], alp[kMaxAnc];  // b and a of the ancestor at depth e
    alp[0] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a0), 0));
    bet[0] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(b0), 0));
    float g = alp[0];
    unsigned long long mm = m;
#pragma unroll
    for (int e = 1; e <= kMaxP; ++e) {
      const int a = imin((int)__ffsll((long long)mm), nl);  // 0 (the root) beyond the depth
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
    // W1[t, anc e] = cwl[e] z[e] with cwl[e] = b_{anc e} g_t / g_{anc e}
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
  if constexpr (CM) {
    if (tw == 0) cm_walk();
  }
  __builtin_amdgcn_s_waitcnt(0);  // vmcnt(0) lgkmcnt(0): rows landed, prologue written
  wg_barrier();   // (1) rows, masks, gates and cleared regions are in LDS

  // ---- Gram tiles [Q; K] K^T of the lower node triangle, dealt between the tree waves ----
  // Transposed: lane (g, t) owns node t = 16 mt + l16 and gets k_s . k_t and k_s . q_t for
  // s = 16 nt + 4 g + 0..3.  Entries of ancestor pairs are kept at depth(s) = (t's
  // ancestors-or-self in slots 0..s) - 1 (the k.k ones times b_t, the factor the path solve
  // applies); the rest go to padding entries 17..19.  Rows past the node count read finite
  // or arbitrary LDS contents; the entries they produce are never kept.
  const int ntg = (n + 15) / 16;
#pragma unroll
  for (int mt = 0; mt < NTG; ++mt) {
#pragma unroll
    for (int nt = 0; nt <= mt; ++nt) {
      if ((mt * (mt + 1) / 2 + nt) % kTreeWaves != kTreeWaves - 1 - tw || mt >= ntg) continue;
      const int tme = 16 * mt + l16, ra = imin(tme, nl);
      const int rbr = 16 * nt + l16;
      f32x4 gk4 = {0.f, 0.f, 0.f, 0.f}, gq4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        bf16x8 aqh, aqm, aql, akh, akm, akl, bh, bm, bl;
        row_frag<D, BF16IN>(qrow, tme, 32 * ks + 8 * g4, aqh, aqm, aql);
        row_frag<D, BF16IN>(krow, tme, 32 * ks + 8 * g4, akh, akm, akl);
        row_frag<D, BF16IN>(krow, rbr, 32 * ks + 8 * g4, bh, bm, bl);
        if constexpr (BF16IN) {
          gk4 = mfma_bf16(bh, akh, gk4);
          gq4 = mfma_bf16(bh, aqh, gq4);
        } else {
          gk4 = mfma_x6(bh, bm, bl, akh, akm, akl, gk4);
          gq4 = mfma_x6(bh, bm, bl, aqh, aqm, aql, gq4);
          drain(gk4);  // the next fragments are split on VALU into the same registers
          drain(gq4);
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
        s.cw[keep ? trow + es : dummy] = gq4[r];
        s.cy[keep && sn != tme ? trow + es : dummy] = gk4[r] * bt;
      }
      // the next tile's fragments are loaded only after these products' results are stored
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  tree_sync(&s.sync, &s.bad, kTreeWaves, lane);  // the compact Gram rows are complete

  // ---- tw 0: path solve, one lane per node, then the node's compact W1 row ---------------
  // Writes -g_t Y[t, e] over the k.k entries and W1[t, e] over the q.k entries: every read of
  // them (this wave's, in program order) comes first.
  if (tw == 0) {
    const bool tv = t_me < n;
    const int t = tn;
    const int dmax = wave_max_i32(tv ? d_me : 0);
    const float z_root = s.cw[0];  // q_0 . k_0
    auto anc_at = [&](int e) -> int { return (int)((ancw[e >> 2] >> (8 * (e & 3))) & 0xffu); };
    float z[kAR];  // right-hand side q_t . k_{anc e}; zero beyond the depth
#pragma unroll
    for (int v = 0; v < kAR / 4; ++v) {
      const float4 x = reinterpret_cast<const float4 *>(&s.cw[t * kAR])[v];
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
        const float4 *row = reinterpret_cast<const float4 *>(&s.cy[anc_at(e2) * kAR]);
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
      for (int e = 0; e <= kMaxP; ++e)
        if (e <= d_me) s.cw[t * kAR + e] = s.cwl[e][lane] * z[e];  // W1[t, e]
    }
    if (lane == 0) s.cw[0] = s.beta[0] * z_root;  // the root: W1[0, 0] = b_0 (q_0 . k_0)
  }
  tree_sync(&s.sync, &s.bad, 2 * kTreeWaves, lane);  // the compact W1 rows are written
  __builtin_amdgcn_s_setprio(1);  // the chain is done; the product waves' U and W1 U go first
  const int tt = tid - 64 * NPW;
  bf16x8 fh[PXN], fm[PXN], fl[PXN];
#pragma unroll
  for (int x = 0; x < PXN; ++x)
    if (tt + 64 * kTreeWaves * x < PIT) fill_item(tt + 64 * kTreeWaves * x, fh[x], fm[x], fl[x]);
  float f64v = 0.f;  // W1[64][lane] on tree wave 0
  if constexpr (X65) {
    if (tw == 0 && row64) {
      const unsigned long long aset = (s.mask[64] << 1) | 1ull;
      const int d = imin((int)__popcll(aset & ((2ull << lane) - 1ull)) - 1, kAR - 1);
      f64v = ((aset >> lane) & 1ull) ? s.cw[64 * kAR + d] : 0.f;
    }
  }
  wg_barrier();  // (2) the compact W1 rows are solved; nobody reads q or k rows any more
#pragma unroll
  for (int x = 0; x < PXN; ++x) {
    const int it = tt + 64 * kTreeWaves * x;
    if (it < PIT) {
      const int off = fill_off(it);
      *reinterpret_cast<uint4 *>(pl + off) = __builtin_bit_cast(uint4, fh[x]);
      *reinterpret_cast<uint4 *>(pl + G::PR * SPD + off) = __builtin_bit_cast(uint4, fm[x]);
      *reinterpret_cast<uint4 *>(pl + 2 * G::PR * SPD + off) = __builtin_bit_cast(uint4, fl[x]);
    }
  }
  if constexpr (X65) {
    if (tw == 0 && row64) s.w64[lane] = f64v;
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the dense W1 rows are written
  wg_barrier();  // (3) the dense W1 rows are ready
  if (!stage_v) wg_barrier();  // (3b) the dense W1 rows are read
  wg_barrier();  // (4) every output row is staged
  store_rows();
}

template <int D, bool BF16IN, int NT, bool X65>
hipError_t launch_one(const VerifyParams &p, hipStream_t stream) {
  const unsigned units = (unsigned)(p.L * p.B * p.H);
  if (p.pv_parent)
    hipLaunchKernelGGL((verify_kernel<D, BF16IN, NT, X65, true>), dim3(units),
                       dim3(VerifyGeom<D, BF16IN, NT, X65>::NTH), 0, stream, p);
  else
    hipLaunchKernelGGL((verify_kernel<D, BF16IN, NT, X65, false>), dim3(units),
                       dim3(VerifyGeom<D, BF16IN, NT, X65>::NTH), 0, stream, p);
  return hipGetLastError();
}

template <int D, bool BF16IN>
hipError_t launch_nt(const VerifyParams &p, hipStream_t stream) {
  if (p.R == kMaxSlots) return launch_one<D, BF16IN, 4, true>(p, stream);
  switch ((p.R + 15) / 16) {
    case 1: return launch_one<D, BF16IN, 1, false>(p, stream);
    case 2: return launch_one<D, BF16IN, 2, false>(p, stream);
    case 3: return launch_one<D, BF16IN, 3, false>(p, stream);
    default: return launch_one<D, BF16IN, 4, false>(p, stream);
  }
}

}  // namespace

hipError_t launch_verify(const VerifyParams &p, hipStream_t stream) {
  if (p.D == 64) return p.in_bf16 ? launch_nt<64, true>(p, stream) : launch_nt<64, false>(p, stream);
  return p.in_bf16 ? launch_nt<128, true>(p, stream) : launch_nt<128, false>(p, stream);
}

}  // namespace gdntree
