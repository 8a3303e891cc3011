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
  static constexpr int CH = 16 / (int)sizeof(T);        // elements per 16-byte chunk
  static constexpr int CPR = D / CH;                     // chunks per row
  static constexpr int SP = (16 * NT + 31) / 32 * 32;    // node axis padded for MFMA k-steps
  static constexpr int DS = SP + 8;                      // dense W row stride (bf16)
  static constexpr int ROWB0 = RM * D * (int)sizeof(T);  // bytes of one matrix's rows
  static constexpr int ROWB = (ROWB0 + 1023) / 1024 * 1024;  // whole 1 KiB load instructions
  static constexpr int REST = 2 * RM * DS * 2 + 3 * RM * kAR * 4 + RM * kAR + RM * 8 + RM * 21 + 64;
  // k, q, v rows of a head; two buffers when they fit, so the next head's rows can arrive
  // (direct global -> LDS loads) while this head is processed.  After the effective-query
  // operands have been gathered, qe_hi and qe_lo (bf16) take the place of the k and v rows.
  static constexpr int NBUF = (2 * 3 * ROWB + REST <= 160 * 1024) ? 2 : 1;
  alignas(16) uint16_t dense[2][RM * DS];                // -W2, later W1 (hi | lo)
  alignas(16) float lc[RM * kAR];                        // k.k Gram -> Lm rows
  alignas(16) float mc[RM * kAR];                        // q.k Gram -> Mm rows
  alignas(16) float wc[RM * kAR];                        // W1 rows (compact, by depth)
  alignas(16) int8_t anc[RM * kAR];                      // ancestor slot at each depth
  alignas(16) unsigned long long mask[RM];
  float alpha[RM], beta[RM], gamma[RM];
  int parent[RM];
  int8_t depth[RM];
  int bad;
};

// Workgroup barrier that orders LDS accesses only.  __syncthreads() also waits for every
// direct-to-LDS load still in flight, i.e. for the next head's rows, which would serialize
// the prefetch with this head's work.  The phases exchange data through LDS alone, and the
// next head's rows are waited for explicitly before they are read.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt left alone
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The k, q, v rows of one head.  The two row buffers are separate LDS objects so that the
// compiler can tell the buffer being read from the one the next head's loads are filling
// (it otherwise waits for those loads before every LDS access).
template <int ROWB>
struct RowBuf {
  alignas(16) unsigned char m[3][ROWB];
};

// Rows live in LDS unpadded with their 16-byte chunks XOR-swizzled by the row index, so that
// 16 consecutive rows read at the same logical column hit distinct banks.
template <int D, int CH>
__device__ __forceinline__ int swz(int r, int i) {
  constexpr int CPR = D / CH;
  return r * D + ((((i / CH) ^ (r & (CPR - 1)))) * CH) + (i % CH);
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void gbl_void_t;

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

// One 16x16 Gram tile (k-steps over d_k) between swizzled LDS rows ra of A and rb of B.
template <int D, bool BF16IN>
__device__ __forceinline__ f32x4 gram_tile(const typename InT<BF16IN>::T *A,
                                           const typename InT<BF16IN>::T *Bm, int ra, int rb, int kofs) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    const int col = 32 * ks + kofs;
    if constexpr (BF16IN) {
      acc = mfma(lds_frag(A + swz<D, 8>(ra, col)), lds_frag(Bm + swz<D, 8>(rb, col)), acc);
    } else {
      float ya[8], yb[8];  // two swizzled 4-float chunks per operand
      const float4 a0 = *reinterpret_cast<const float4 *>(A + swz<D, 4>(ra, col));
      const float4 a1 = *reinterpret_cast<const float4 *>(A + swz<D, 4>(ra, col + 4));
      const float4 b0 = *reinterpret_cast<const float4 *>(Bm + swz<D, 4>(rb, col));
      const float4 b1 = *reinterpret_cast<const float4 *>(Bm + swz<D, 4>(rb, col + 4));
      ya[0] = a0.x; ya[1] = a0.y; ya[2] = a0.z; ya[3] = a0.w; ya[4] = a1.x; ya[5] = a1.y; ya[6] = a1.z; ya[7] = a1.w;
      yb[0] = b0.x; yb[1] = b0.y; yb[2] = b0.z; yb[3] = b0.w; yb[4] = b1.x; yb[5] = b1.y; yb[6] = b1.z; yb[7] = b1.w;
      bf16x8 ah, al, bh, bl;
      split8(ya, ah, al);
      split8(yb, bh, bl);
      acc = mfma(ah, bh, acc);
      acc = mfma(al, bh, acc);
      acc = mfma(ah, bl, acc);
    }
  }
  return acc;
}

// Persistent tree-verify kernel.  A workgroup of W waves owns 16*W value channels of a head
// (all of them when W = D/16) and loops over heads.  While it works on one head, the next
// head's k, q and v rows are already arriving in the other LDS row buffer (direct global ->
// LDS loads, no registers), so HBM traffic overlaps the tree prologue and the MFMA work.
// Every wave issues a fixed number of those loads (padded buffers, clamped sources), which
// keeps the compiler's memory-counter waits exact: waiting for this head's S0^T fragments
// never waits for the next head's rows.  Each wave owns one 16-channel tile of d_v (its rows
// of S0^T) and the d_k tiles wave, wave + W, ... of the effective queries.
template <int D, bool BF16IN, int NT, int W, int JT>
__global__ __launch_bounds__(64 * W, 1) void verify_kernel(VerifyParams p, int units) {
  typedef VerifySmem<D, BF16IN, NT> SM;
  typedef typename SM::T T;
  constexpr int RM = SM::RM, DS = SM::DS, CH = SM::CH, CPR = SM::CPR;
  constexpr int KS = D / 32;          // MFMA k-steps over d_k
  constexpr int KSS = SM::SP / 32;    // MFMA k-steps over the node axis
  constexpr int nthr = 64 * W;
  constexpr int S = D / (16 * W * JT);  // value-channel slices per head
  constexpr int NI = D / 16;          // 16-channel tiles of d_k
  constexpr int RI = (NI + W - 1) / W;
  constexpr int MPT = (RM + nthr - 1) / nthr;     // nodes per thread
  constexpr int QMAX = SM::ROWB / 1024;           // 1 KiB load instructions per matrix
  constexpr int QW = (QMAX + W - 1) / W;          // ... per wave
  constexpr bool DB = SM::NBUF == 2;
  typedef RowBuf<SM::ROWB> RB;
  __shared__ SM s;
  __shared__ RB rbA;
  __shared__ RowBuf<DB ? SM::ROWB : 16> rbB;

  int tid = threadIdx.x, lane = tid & 63, g4 = lane >> 4, l16 = lane & 15;
  const int wave = tid >> 6;
  // Lane-derived indices are re-materialised at every phase boundary: left to itself the
  // compiler hoists every address out of the persistent loop and keeps it live (spilled)
  // across all phases.
#define GDNTREE_FRESH_LANE() asm volatile("" : "+v"(tid), "+v"(lane), "+v"(g4), "+v"(l16))
  const int HT = p.L * p.B * p.H;
  const int G = gridDim.x;
  const T *gq = static_cast<const T *>(p.q);
  const T *gk = static_cast<const T *>(p.k);
  const T *gv = static_cast<const T *>(p.v);
  const T *ga = static_cast<const T *>(p.alpha);
  const T *gb = static_cast<const T *>(p.beta);

  struct Unit {
    int hh, js, h, b, n;
    size_t rowbase;
  };
  auto unit_of = [&](int u) {
    Unit x;
    if (S == 1) {
      x.hh = u;
      x.js = 0;
    } else {  // keep a head's slices on one XCD (workgroups are dealt round-robin to 8 XCDs)
      const int xcd = u & 7, loc = u >> 3;
      x.js = loc % S;
      x.hh = (loc / S) * 8 + xcd;
    }
    const bool in = u < units && x.hh < HT;
    if (!in) {  // a placeholder for loads that keep the instruction count fixed
      x.hh = 0;
      x.js = 0;
    }
    x.h = x.hh % p.H;
    const int lb = x.hh / p.H;
    x.b = lb % p.B;
    x.rowbase = (size_t)lb * p.R;
    // n_nodes is read-only here: a scalar load, so that using it never waits for the
    // vector memory loads in flight (this head's S0^T, the next head's rows)
    const int32_t __attribute__((address_space(4))) *nn_c =
        (const int32_t __attribute__((address_space(4))) *)p.n_nodes;
    const int nv = nn_c[in ? x.b : 0];
    x.n = in ? nv : 0;
    return x;
  };
  auto valid = [&](const Unit &x) { return x.n >= 1 && x.n <= p.R; };
  auto nload = [&](const Unit &x) { return (x.n >= 1 && x.n <= p.R) ? x.n : 1; };

  // Direct global -> LDS loads of a unit's k, q, v rows into row buffer `bi`: each wave
  // instruction fills 64 consecutive 16-byte chunks; lane l of instruction q holds physical
  // chunk 64 q + l and fetches the logical chunk that the swizzle places there.  Chunks of
  // rows past the unit's node count (and of the padding) fetch a valid row and are never read.
  auto issue_rows = [&](const Unit &x, auto &rb) {
    const int nn = nload(x);
#pragma unroll
    for (int m = 0; m < 3; ++m) {
      const T *g = m == 0 ? gk : m == 1 ? gq : gv;
      unsigned char *dst = rb.m[m];
      // buffer (not global) loads: the compiler then keeps exact counts of the loads in
      // flight, so waiting for this head's S0^T does not wait for these rows
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          (void *)(g + (x.rowbase * p.H + x.h) * (size_t)D), 0, nn * p.H * D * (int)sizeof(T),
          0x00020000);
#pragma unroll
      for (int k = 0; k < QW; ++k) {
        const int qi = min(wave + k * W, QMAX - 1);
        const int pc = 64 * qi + lane, r = pc / CPR, c = (pc % CPR) ^ (r & (CPR - 1));
        const unsigned off = (unsigned)((min(r, nn - 1) * p.H * D + c * CH) * (int)sizeof(T));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t *)(dst + 1024 * qi), 16, off, 0, 0, 0);
      }
    }
  };
  int m_par[MPT];
  unsigned long long m_mask[MPT];
  float m_al[MPT], m_be[MPT];
  auto prefetch_meta = [&](const Unit &x) {
    const int nn = nload(x);
#pragma unroll
    for (int i = 0; i < MPT; ++i) {
      const int t = min(tid + i * nthr, nn - 1);
      m_par[i] = p.parent[(size_t)x.b * p.R + t];
      m_mask[i] = p.anc[(size_t)x.b * p.R + t];
      const size_t gi = (x.rowbase + t) * p.H + x.h;
      m_al[i] = load_elem(ga, gi);
      m_be[i] = load_elem(gb, gi);
    }
  };

  int u = blockIdx.x;
  Unit cur = unit_of(u);
  if (DB) issue_rows(cur, rbA);
  prefetch_meta(cur);
  Unit nxt = unit_of(u + G);

  // One unit: its rows are in `crb`; the next unit's rows go to `nrb`.
  auto step = [&](auto &crb, auto &nrb) {
    GDNTREE_FRESH_LANE();
    const int n = cur.n;
    const bool live = valid(cur);
    const int h = cur.h, js = cur.js;
    auto row_off = [&](int t) -> size_t { return ((cur.rowbase + t) * p.H + h) * (size_t)D; };
    const int j0 = (js * W + wave) * 16 * JT;  // this wave's JT tiles of 16 value channels
    T *Kr = reinterpret_cast<T *>(crb.m[0]);
    T *Qr = reinterpret_cast<T *>(crb.m[1]);
    T *Vr = reinterpret_cast<T *>(crb.m[2]);
    uint16_t *Qhi = reinterpret_cast<uint16_t *>(crb.m[0]);  // over the k rows
    uint16_t *Qlo = reinterpret_cast<uint16_t *>(crb.m[2]);  // over the v rows

    // ---- 0. this unit's rows and metadata; S0^T fragments; the next unit's loads ------
    if (!DB) issue_rows(cur, crb);
    __builtin_amdgcn_s_waitcnt(0);  // rows (and metadata) of this unit have landed
    if (live) {
      if (tid == 0) s.bad = 0;
#pragma unroll
      for (int i = 0; i < MPT; ++i) {
        const int t = tid + i * nthr;
        if (t < n) {
          s.parent[t] = m_par[i];
          s.mask[t] = m_mask[i];
          s.alpha[t] = m_al[i];
          s.beta[t] = m_be[i];
        }
      }
    }
    f32x4 sc[JT][KS][2];
#pragma unroll
    for (int jt = 0; jt < JT; ++jt) {
      const float *sb = p.state + (size_t)cur.hh * D * D + (size_t)(j0 + 16 * jt + l16) * D + 8 * g4;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        sc[jt][ks][0] = *reinterpret_cast<const f32x4 *>(sb + 32 * ks);
        sc[jt][ks][1] = *reinterpret_cast<const f32x4 *>(sb + 32 * ks + 4);
      }
    }
    const Unit after = unit_of(u + 2 * G);
    __syncthreads();  // every wave's part of this buffer has landed; the other one is free
    if (DB) issue_rows(nxt, nrb);
    prefetch_meta(nxt);

    GDNTREE_FRESH_LANE();
    // ---- 1a. per node: validate links, ancestors from the bitmask, path gate ------------
    if (live) {
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
      // ---- 1b. Gram entries k_t.k_s and q_t.k_s for s ancestor-or-self of t (MFMA) ------
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
        const f32x4 g = gram_tile<D, BF16IN>(Kr + part * (SM::ROWB / (int)sizeof(T)), Kr, ra, rb, 8 * g4);
        const int sn = 16 * nt + l16;
        const int es = __popcll(s.mask[rb]);
        float *dst = s.lc + part * (int)(s.mc - s.lc);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 16 * mt + 4 * g4 + r;
          const unsigned long long mtt = s.mask[min(t, n - 1)];
          const bool anc = sn == 0 || ((mtt >> (sn - 1)) & 1ull);
          if (t < n && sn <= t && es <= kMaxP && anc) dst[t * kAR + es] = g[r];
        }
      }
    }
    lds_barrier();
    const bool bad = live && s.bad;
    const bool work = live && !bad;

    GDNTREE_FRESH_LANE();
    // ---- 2. per node: Lm, Mm rows; then the Wm solve; W1 rows and the dense -W2 ---------
    if (work) {
      for (int t = tid; t < n; t += nthr) {
        const int dt = s.depth[t];
        int arow[kAR];
        load_anc20(&s.anc[t * kAR], arow);
        float gk2[kAR], gqk[kAR];
        load_row20(&s.lc[t * kAR], gk2);
        load_row20(&s.mc[t * kAR], gqk);
        const float bt = s.beta[t];
        float rho = 1.f;  // g_t / g_{anc at depth e}
        float lrow[kAR], mrow[kAR];
#pragma unroll
        for (int e = kAR - 1; e >= 0; --e) {
          const bool on = e < kA && e <= dt;
          mrow[e] = on ? rho * gqk[e] : 0.f;
          lrow[e] = (e < dt) ? bt * rho * gk2[e] : 0.f;
          const float ae = (e < kA) ? s.alpha[arow[e]] : 1.f;
          rho *= on ? ae : 1.f;
        }
        store_row20(&s.lc[t * kAR], lrow);
        store_row20(&s.mc[t * kAR], mrow);
      }
    }
    lds_barrier();
    GDNTREE_FRESH_LANE();
    if (work) {
      for (int t = tid; t < n; t += nthr) {
        const int dt = s.depth[t];
        // ancestor slots stay packed four to a word and are unpacked where used
        const uint4 ap = *reinterpret_cast<const uint4 *>(&s.anc[t * kAR]);
        const uint32_t ap4 = *reinterpret_cast<const uint32_t *>(&s.anc[t * kAR + 16]);
        auto anc_at = [&](int e) -> int {
          const uint32_t wd = e < 4 ? ap.x : e < 8 ? ap.y : e < 12 ? ap.z : e < 16 ? ap.w : ap4;
          return (int)((wd >> (8 * (e & 3))) & 0xffu);
        };
        float w[kAR];
        load_row20(&s.mc[t * kAR], w);  // Mm row, zero beyond the depth
        // right-looking solve of w (I + Lm) = Mm over the path, deepest ancestor first; for
        // depths beyond dt, w is zero and the ancestor slot is the root, whose Lm row is zero
        // (two ancestor rows in flight at a time: the scheduler barriers keep the loads of
        // later rows from being hoisted, which would need a register per entry)
#pragma unroll
        for (int grp = 0; grp < kMaxP / 2; ++grp) {
          float lr[2][16];
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int e2 = kMaxP - 2 * grp - q;
            const float4 *row = reinterpret_cast<const float4 *>(&s.lc[anc_at(e2) * kAR]);
#pragma unroll
            for (int v = 0; v < (e2 + 3) / 4; ++v) {
              const float4 x = row[v];
              lr[q][4 * v] = x.x; lr[q][4 * v + 1] = x.y; lr[q][4 * v + 2] = x.z; lr[q][4 * v + 3] = x.w;
            }
          }
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int e2 = kMaxP - 2 * grp - q;
#pragma unroll
            for (int e = 0; e < e2; ++e) w[e] -= w[e2] * lr[q][e];
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        int arow[kAR];
#pragma unroll
        for (int e = 0; e < kAR; ++e) arow[e] = anc_at(e);
        float w1[kAR];
        uint16_t *dh = s.dense[0] + t * DS, *dl = s.dense[1] + t * DS;
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
    }
    lds_barrier();

    GDNTREE_FRESH_LANE();
    // ---- 3. effective queries: qe^T = g q^T - K^T W2^T (MFMA), split hi/lo (bf16) --------
    // First every K^T and V^T operand fragment is gathered from the k and v rows; after a
    // barrier qe_hi and qe_lo overwrite those rows.
    bf16x8 kt_hi[RI][KSS], kt_lo[RI][KSS];  // K^T: this wave's d_k tiles, node slots
    bf16x8 vt_hi[JT][KSS], vt_lo[JT][KSS];  // V^T: this wave's value channels, node slots
    if (work) {
#pragma unroll
      for (int kk = 0; kk < KSS; ++kk) {
#pragma unroll
        for (int r = 0; r < RI; ++r) {
          const int it = wave + r * W;
          if (it < NI) {
            if constexpr (BF16IN) {
              u16x8 f;
#pragma unroll
              for (int x = 0; x < 8; ++x) f[x] = Kr[swz<D, CH>(min(32 * kk + 8 * g4 + x, n - 1), 16 * it + l16)];
              kt_hi[r][kk] = __builtin_bit_cast(bf16x8, f);
            } else {
              float f[8];
#pragma unroll
              for (int x = 0; x < 8; ++x) f[x] = Kr[swz<D, CH>(min(32 * kk + 8 * g4 + x, n - 1), 16 * it + l16)];
              split8(f, kt_hi[r][kk], kt_lo[r][kk]);
            }
          }
        }
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) {
          const int col = j0 + 16 * jt + l16;
          if constexpr (BF16IN) {
            u16x8 f;
#pragma unroll
            for (int x = 0; x < 8; ++x) f[x] = Vr[swz<D, CH>(min(32 * kk + 8 * g4 + x, n - 1), col)];
            vt_hi[jt][kk] = __builtin_bit_cast(bf16x8, f);
          } else {
            float f[8];
#pragma unroll
            for (int x = 0; x < 8; ++x) f[x] = Vr[swz<D, CH>(min(32 * kk + 8 * g4 + x, n - 1), col)];
            split8(f, vt_hi[jt][kk], vt_lo[jt][kk]);
          }
        }
      }
    }
    lds_barrier();  // k and v rows are dead: qe_hi and qe_lo take their place
    GDNTREE_FRESH_LANE();
    if (work) {
      const int ntiles = (n + 15) / 16;
#pragma unroll
      for (int r = 0; r < RI; ++r) {
        const int it = wave + r * W;  // d_k tile of 16 channels
        if (it >= NI) break;
        const int i = 16 * it + 4 * g4;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          if (nt >= ntiles) break;
          const int t = 16 * nt + l16, tb = min(t, n - 1);
          const float gt = s.gamma[tb];
          f32x4 acc;
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[e] = gt * load_elem(Qr, (size_t)swz<D, CH>(tb, i + e));
#pragma unroll
          for (int kk = 0; kk < KSS; ++kk) {
            const bf16x8 bh = lds_frag(s.dense[0] + tb * DS + 32 * kk + 8 * g4);
            const bf16x8 bl = lds_frag(s.dense[1] + tb * DS + 32 * kk + 8 * g4);
            acc = mfma(kt_hi[r][kk], bh, acc);
            acc = mfma(kt_hi[r][kk], bl, acc);
            if constexpr (!BF16IN) acc = mfma(kt_lo[r][kk], bh, acc);
          }
          if (t < n) {
            typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
            bf16x4 hv, lv;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              hv[e] = (__bf16)acc[e];
              lv[e] = (__bf16)(acc[e] - (float)hv[e]);
            }
            *reinterpret_cast<bf16x4 *>(Qhi + swz<D, 8>(t, i)) = hv;
            *reinterpret_cast<bf16x4 *>(Qlo + swz<D, 8>(t, i)) = lv;
          }
        }
      }
    }
    lds_barrier();
    GDNTREE_FRESH_LANE();
    // the dense W1 (hi | lo) replaces -W2
    if (work) {
      for (int t = tid; t < n; t += nthr) {
        int arow[kAR];
        load_anc20(&s.anc[t * kAR], arow);
        float w1[kAR];
        load_row20(&s.wc[t * kAR], w1);
        uint16_t *dh = s.dense[0] + t * DS, *dl = s.dense[1] + t * DS;
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
    }
    lds_barrier();

    GDNTREE_FRESH_LANE();
    // ---- 4. o^T = S0^T [qe] + V^T W1^T (MFMA), node tile by node tile --------------------
    if (work) {
      bf16x8 ahi[JT][KS], alo[JT][KS];
#pragma unroll
      for (int jt = 0; jt < JT; ++jt)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const float x[8] = {sc[jt][ks][0][0], sc[jt][ks][0][1], sc[jt][ks][0][2], sc[jt][ks][0][3],
                              sc[jt][ks][1][0], sc[jt][ks][1][1], sc[jt][ks][1][2], sc[jt][ks][1][3]};
          split8(x, ahi[jt][ks], alo[jt][ks]);
        }
      const int ntiles = (n + 15) / 16;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        if (nt >= ntiles) break;
        const int t = 16 * nt + l16;
        const int tb = min(t, n - 1);
        f32x4 acc0[JT], acc1[JT];
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) {
          acc0[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
          acc1[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {  // S0^T qe: hi*hi into acc0, cross terms into acc1
          const int col = 32 * ks + 8 * g4;
          const bf16x8 bhi = lds_frag(Qhi + swz<D, 8>(tb, col));
          const bf16x8 blo = lds_frag(Qlo + swz<D, 8>(tb, col));
#pragma unroll
          for (int jt = 0; jt < JT; ++jt) {
            acc0[jt] = mfma(ahi[jt][ks], bhi, acc0[jt]);
            acc1[jt] = mfma(alo[jt][ks], bhi, acc1[jt]);
            acc1[jt] = mfma(ahi[jt][ks], blo, acc1[jt]);
          }
        }
#pragma unroll
        for (int kk = 0; kk < KSS; ++kk) {  // V^T W1^T over the node axis
          const bf16x8 wh = lds_frag(s.dense[0] + tb * DS + 32 * kk + 8 * g4);
          const bf16x8 wl = lds_frag(s.dense[1] + tb * DS + 32 * kk + 8 * g4);
#pragma unroll
          for (int jt = 0; jt < JT; ++jt) {
            acc0[jt] = mfma(vt_hi[jt][kk], wh, acc0[jt]);
            acc1[jt] = mfma(vt_hi[jt][kk], wl, acc1[jt]);
            if constexpr (!BF16IN) acc1[jt] = mfma(vt_lo[jt][kk], wh, acc1[jt]);
          }
        }
        if (t < n) {
#pragma unroll
          for (int jt = 0; jt < JT; ++jt) {
            const size_t ob = row_off(t) + j0 + 16 * jt + 4 * g4;
            const f32x4 o = acc0[jt] + acc1[jt];
            if (p.out_bf16) {
              typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
              const bf16x4 ob4 = {(__bf16)o[0], (__bf16)o[1], (__bf16)o[2], (__bf16)o[3]};
              *reinterpret_cast<bf16x4 *>(static_cast<uint16_t *>(p.o) + ob) = ob4;
            } else {
              *reinterpret_cast<f32x4 *>(static_cast<float *>(p.o) + ob) = o;
            }
          }
        }
      }
    }
    if (bad) {  // an inconsistent tree: NaN outputs for this request (after all loads)
      const int jw0 = js * 16 * W * JT, span = 16 * W * JT;
      for (int c = tid; c < n * span; c += nthr) {
        const size_t oi = row_off(c / span) + jw0 + c % span;
        if (p.out_bf16) static_cast<uint16_t *>(p.o)[oi] = 0x7fc0;
        else static_cast<float *>(p.o)[oi] = __builtin_nanf("");
      }
    }
    lds_barrier();  // LDS is rewritten for the next unit
    cur = nxt;
    nxt = after;
    u += G;
  };
  // unrolled by two so that each half names its buffers statically
  while (u < units) {
    step(rbA, rbB);
    if (u >= units) break;
    if constexpr (DB) step(rbB, rbA);
    else step(rbA, rbA);
  }
#undef GDNTREE_FRESH_LANE
}

template <int D, bool BF16IN, int NT, int W, int JT>
hipError_t launch_w(const VerifyParams &p, hipStream_t stream) {
  const int HT = p.L * p.B * p.H;
  constexpr int S = D / (16 * W * JT);
  const int units = (S == 1) ? HT : ((HT + 7) / 8) * 8 * S;
  int grid = units;
  if (S == 1) {  // persistent: one workgroup per CU, each looping over heads
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0)
      grid = min(units, cus);
  }
  hipLaunchKernelGGL((verify_kernel<D, BF16IN, NT, W, JT>), dim3((unsigned)grid), dim3(64 * W), 0, stream,
                     p, units);
  return hipGetLastError();
}

// A whole head per workgroup (four waves, each owning D/64 tiles of 16 value channels) when
// there are enough heads to occupy the chip; otherwise a head's value channels are split
// over several workgroups.
template <int D, bool BF16IN, int NT>
hipError_t launch_one(const VerifyParams &p, hipStream_t stream) {
  const int HT = p.L * p.B * p.H;
  if (HT >= 64) return launch_w<D, BF16IN, NT, 4, D / 64>(p, stream);
  return launch_w<D, BF16IN, NT, D / 64, 1>(p, stream);
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
