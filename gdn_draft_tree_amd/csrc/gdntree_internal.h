// Internal declarations shared by the gfx950 kernels and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/gdntree.h"

namespace gdntree {

constexpr int kMaxN = 64;          // draft nodes
constexpr int kMaxSlots = kMaxN + 1;
constexpr int kMaxP = 16;          // positions, hence tree depth
constexpr int kMaxK = 64;          // candidates per position
constexpr int kMaxAnc = kMaxP + 1; // ancestors-or-self of a node (depth 0..16)
constexpr int kCondMaxK = 16;      // candidates per position with parent-conditioned rows
constexpr int kSharedMaxSlots = 4096;  // keys the budget cut holds: pow2(B) * min(N, G)
constexpr int kSharedMaxB = 1024;      // requests of a build under a shared budget

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

// Element loads for the two input dtypes.
__device__ __forceinline__ float load_elem(const uint16_t *p, size_t i) { return bf16_bits_to_f32(p[i]); }
__device__ __forceinline__ float load_elem(const float *p, size_t i) { return p[i]; }

// Launchers (defined next to their kernels).  They assume validated arguments.
hipError_t launch_build(const float *lat_logp, const int32_t *lat_tok, const int32_t *root_tok,
                        int B, int P, int K, int N, gdntree_tree out, hipStream_t stream);

// best-first build over parent-conditioned edge log-probs [B][P][K][K] (K <= kCondMaxK)
hipError_t launch_build_cond(const float *edge_logp, const int32_t *lat_tok, const int32_t *root_tok, int B,
                             int P, int K, int N, gdntree_tree out, hipStream_t stream);
// Markov-head edge log-probs [B][P][K][K] from base logits, token ids and the head's embeddings
hipError_t launch_markov_edges(const float *bases, const int32_t *lat_tok, const int32_t *root_tok,
                               const void *W1, const void *W2, bool w_bf16, int B, int P, int K, int V, int R,
                               float *edge_logp, hipStream_t stream);

struct VerifyParams {
  const int32_t *parent;
  const unsigned long long *anc;
  const int32_t *n_nodes;
  const void *q, *k, *v, *alpha, *beta;
  const float *state;
  void *o;
  int B, R, L, H, D;   // R = N + 1 slots
  int in_bf16, out_bf16;
  // The previous step's acceptance and commit, done by the same launch before the verify
  // (pv_parent == nullptr: none).  The previous tree, its target argmax and its rows (same
  // layer, request, head and dtype layout, pv_R = previous N + 1 slots); the state is then
  // written in place through `state`.  acc_*: the acceptance, written when non-null.
  const int32_t *pv_parent = nullptr, *pv_token = nullptr, *pv_n_nodes = nullptr, *pv_target = nullptr;
  const void *pv_k = nullptr, *pv_v = nullptr, *pv_alpha = nullptr, *pv_beta = nullptr;
  int32_t *acc_len = nullptr, *acc_tok = nullptr, *acc_node = nullptr;
  int pv_R = 0, pv_P = 0;
};
hipError_t launch_verify(const VerifyParams &p, hipStream_t stream);

struct CommitParams {
  const int32_t *parent, *token, *n_nodes, *target;  // target: acceptance only
  const void *k, *v, *alpha, *beta;
  float *state;
  int32_t *acc_len, *acc_tok, *acc_node;
  int B, R, P, L, H, D;
  int in_bf16;
};
hipError_t launch_accept_commit(const CommitParams &p, hipStream_t stream);
hipError_t launch_accept(const CommitParams &p, hipStream_t stream);  // acceptance only
hipError_t launch_commit(const CommitParams &p, hipStream_t stream);  // commit of a given path
struct BuildParams;
hipError_t launch_build_params(const BuildParams &bp, int B, hipStream_t stream);
// per-request builds, then the cut of every request's node count to a batch budget of G drafts
hipError_t launch_build_shared(const BuildParams &bp, int B, int G, hipStream_t stream);
int shared_budget_lists(int B);  // B rounded up to a power of two
// the cut alone, for trees already built per request (capped at N)
hipError_t launch_budget_cut(const gdntree_tree &out, int B, int N, int G, hipStream_t stream);
// commit of a given path (p) fused with the build of nb other requests' trees (bp)
hipError_t launch_commit_build(const CommitParams &p, const BuildParams &bp, int nb, hipStream_t stream);
// acceptance (written to p.acc_*), commit and the build of nb next trees in one launch
hipError_t launch_accept_commit_build(const CommitParams &p, const BuildParams &bp, int nb, hipStream_t stream);

}  // namespace gdntree
