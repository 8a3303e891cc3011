// Parent-conditioned edge log-probs of a DSpark-style Markov head on gfx950.
//
// The head scores candidate y at position s as l_s(y) = bases(y) + <W1[x_{s-1}], W2[y]>,
// x_{s-1} the previous token (SpecPilot summary, Prerequisites > parallel drafters and
// lattices).  In a draft tree a child's previous token is its parent's: the root token at
// position 0, else the parent's candidate at position s-1.  The edge log-prob is l_s minus the
// log-sum-exp of l_s over the position's K candidates.
//
// One workgroup per (request, position): the rows of W1 (the K previous tokens, or the root
// token alone) and of W2 (the K candidates) are gathered into LDS once, then one wave per
// previous-token row forms the K logits (lane r: candidate r, an fp32 dot product over R) and
// their log-softmax (max-shifted, wave reductions).  All arithmetic is fp32.

#include "gdntree_internal.h"

namespace gdntree {
namespace {

constexpr int kMarkovMaxR = 64;

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Element j of row x of a [V][R] matrix through a buffer resource covering the matrix: a
// token id outside [0, V) gives an offset past the range, which reads zero.
template <bool BF16W>
__device__ __forceinline__ float w_elem(__amdgpu_buffer_rsrc_t rs, int x, int j, int V, int R) {
  const unsigned long long e = (unsigned long long)(unsigned)x * (unsigned)R + (unsigned)j;
  const bool in = x >= 0 && x < V;
  if constexpr (BF16W) {
    const unsigned off = in ? (unsigned)(2 * e) : (unsigned)(2ull * V * R);
    const unsigned short h = __builtin_amdgcn_raw_buffer_load_b16(rs, (int)off, 0, 0);
    return __uint_as_float((unsigned)h << 16);
  } else {
    const unsigned off = in ? (unsigned)(4 * e) : (unsigned)(4ull * V * R);
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, (int)off, 0, 0));
  }
}

template <bool BF16W>
__global__ __launch_bounds__(256) void markov_edges_kernel(const float *bases, const int32_t *lat_tok,
                                                           const int32_t *root_tok, const void *W1, const void *W2,
                                                           int P, int K, int V, int R, float *edge) {
  __shared__ float s_w1[kMaxK][kMarkovMaxR + 1];  // padded rows: lanes along candidates hit distinct banks
  __shared__ float s_w2[kMaxK][kMarkovMaxR + 1];
  __shared__ float s_base[kMaxK];
  const int bs = blockIdx.x, b = bs / P, s = bs - b * P;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t *tok = lat_tok + ((size_t)b * P + s) * K;
  const int nprev = s == 0 ? 1 : K;
  const int wes = BF16W ? 2 : 4;
  const int range = (int)((long long)V * R * wes);
  const __amdgpu_buffer_rsrc_t r1 = __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(W1), 0, range, 0x00020000);
  const __amdgpu_buffer_rsrc_t r2 = __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(W2), 0, range, 0x00020000);
  for (int e = tid; e < nprev * R; e += 256) {
    const int pr = e / R, j = e - pr * R;
    const int x = s == 0 ? root_tok[b] : lat_tok[((size_t)b * P + s - 1) * K + pr];
    s_w1[pr][j] = w_elem<BF16W>(r1, x, j, V, R);
  }
  for (int e = tid; e < K * R; e += 256) {
    const int r = e / R, j = e - r * R;
    s_w2[r][j] = w_elem<BF16W>(r2, tok[r], j, V, R);
  }
  for (int e = tid; e < K; e += 256) s_base[e] = bases[((size_t)b * P + s) * K + e];
  __syncthreads();

  for (int pr = wave; pr < K; pr += 4) {
    const int pw = s == 0 ? 0 : pr;  // at position 0 every row is the root's
    float l = -__builtin_inff();
    if (lane < K) {
      float acc = 0.f;
      for (int j = 0; j < R; ++j) acc = fmaf(s_w1[pw][j], s_w2[lane][j], acc);
      l = s_base[lane] + acc;
    }
    const float m = wave_max(l);
    const float z = wave_sum(lane < K ? expf(l - m) : 0.f);
    if (lane < K) edge[(((size_t)b * P + s) * K + pr) * K + lane] = l - (m + logf(z));
  }
}

}  // namespace

hipError_t launch_markov_edges(const float *bases, const int32_t *lat_tok, const int32_t *root_tok,
                               const void *W1, const void *W2, bool w_bf16, int B, int P, int K, int V, int R,
                               float *edge_logp, hipStream_t stream) {
  if (w_bf16)
    hipLaunchKernelGGL(markov_edges_kernel<true>, dim3(B * P), dim3(256), 0, stream, bases, lat_tok, root_tok, W1,
                       W2, P, K, V, R, edge_logp);
  else
    hipLaunchKernelGGL(markov_edges_kernel<false>, dim3(B * P), dim3(256), 0, stream, bases, lat_tok, root_tok, W1,
                       W2, P, K, V, R, edge_logp);
  return hipGetLastError();
}

}  // namespace gdntree
