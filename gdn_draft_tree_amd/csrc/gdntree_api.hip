// C-ABI entry points: host-side argument validation, then the kernel launches.
// No allocation, no synchronisation, no exceptions across the boundary.

#include <hip/hip_runtime.h>

#include "build_device.h"
#include "gdntree_internal.h"

#define GDNTREE_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

using namespace gdntree;

bool dtype_ok(int d) { return d == GDNTREE_F32 || d == GDNTREE_BF16; }

gdntree_status device_ok() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return GDNTREE_ERR_DEVICE;
  }
  return GDNTREE_OK;
}

gdntree_status head_dims(int dk, int dv) {
  if (dk <= 0 || dv <= 0) return GDNTREE_ERR_ARG;
  if (dk != dv || (dk != 64 && dk != 128)) return GDNTREE_ERR_UNSUPPORTED;
  return GDNTREE_OK;
}

// Grid dimensions must fit in 32 bits: (layers * requests * heads) workgroup units.
bool grid_fits(long long units) { return units > 0 && units * 4 < 0x7fffffffLL; }

}  // namespace

GDNTREE_EXPORT gdntree_status gdntree_build(const float *lat_logp, const int32_t *lat_tok,
                                            const int32_t *root_tok, int B, int P, int K, int N,
                                            gdntree_tree out, hipStream_t stream) {
  if (!lat_logp || !lat_tok || !root_tok || !out.parent || !out.depth || !out.rank ||
      !out.token || !out.score || !out.anc || !out.n_nodes)
    return GDNTREE_ERR_ARG;
  if (B <= 0 || P <= 0 || K <= 0 || N <= 0) return GDNTREE_ERR_ARG;
  if (P > kMaxP || K > kMaxK || N > kMaxN || !grid_fits(B)) return GDNTREE_ERR_UNSUPPORTED;
  if (gdntree_status st = device_ok(); st != GDNTREE_OK) return st;
  if (launch_build(lat_logp, lat_tok, root_tok, B, P, K, N, out, stream) != hipSuccess)
    return GDNTREE_ERR_DEVICE;
  return GDNTREE_OK;
}

GDNTREE_EXPORT gdntree_status gdntree_build_cond(const float *edge_logp, const int32_t *lat_tok,
                                                 const int32_t *root_tok, int B, int P, int K, int N,
                                                 gdntree_tree out, hipStream_t stream) {
  if (!edge_logp || !lat_tok || !root_tok || !out.parent || !out.depth || !out.rank ||
      !out.token || !out.score || !out.anc || !out.n_nodes)
    return GDNTREE_ERR_ARG;
  if (B <= 0 || P <= 0 || K <= 0 || N <= 0) return GDNTREE_ERR_ARG;
  if (P > kMaxP || K > kCondMaxK || N > kMaxN || !grid_fits(B)) return GDNTREE_ERR_UNSUPPORTED;
  if (gdntree_status st = device_ok(); st != GDNTREE_OK) return st;
  if (launch_build_cond(edge_logp, lat_tok, root_tok, B, P, K, N, out, stream) != hipSuccess)
    return GDNTREE_ERR_DEVICE;
  return GDNTREE_OK;
}

GDNTREE_EXPORT gdntree_status gdntree_markov_edges(const float *bases, const int32_t *lat_tok,
                                                   const int32_t *root_tok, const void *W1, const void *W2,
                                                   gdntree_dtype w_dtype, int B, int P, int K, int V, int R,
                                                   float *edge_logp, hipStream_t stream) {
  if (!bases || !lat_tok || !root_tok || !W1 || !W2 || !edge_logp) return GDNTREE_ERR_ARG;
  if (B <= 0 || P <= 0 || K <= 0 || V <= 0 || R <= 0 || !dtype_ok(w_dtype)) return GDNTREE_ERR_ARG;
  const long long wbytes = (long long)V * R * (w_dtype == GDNTREE_BF16 ? 2 : 4);
  if (P > kMaxP || K > kMaxK || R > 64 || wbytes > 0x7fffffffLL || !grid_fits((long long)B * P))
    return GDNTREE_ERR_UNSUPPORTED;
  if (gdntree_status st = device_ok(); st != GDNTREE_OK) return st;
  if (launch_markov_edges(bases, lat_tok, root_tok, W1, W2, w_dtype == GDNTREE_BF16, B, P, K, V, R, edge_logp,
                          stream) != hipSuccess)
    return GDNTREE_ERR_DEVICE;
  return GDNTREE_OK;
}

GDNTREE_EXPORT gdntree_status gdntree_build_shared(const float *lat_logp, const int32_t *lat_tok,
                                                   const int32_t *root_tok, const int32_t *positions,
                                                   int B, int P, int K, int N, int G, gdntree_tree out,
                                                   hipStream_t stream) {
  if (!lat_logp || !lat_tok || !root_tok || !out.parent || !out.depth || !out.rank ||
      !out.token || !out.score || !out.anc || !out.n_nodes)
    return GDNTREE_ERR_ARG;
  if (B <= 0 || P <= 0 || K <= 0 || N <= 0 || G < 0) return GDNTREE_ERR_ARG;
  if (P > kMaxP || K > kMaxK || N > kMaxN || B > kSharedMaxB) return GDNTREE_ERR_UNSUPPORTED;
  // the budget cut holds B (rounded up to a power of two) lists of min(N, G) keys in LDS
  if (G > 0 && (long long)G < (long long)B * N &&
      (long long)shared_budget_lists(B) * (N < G ? N : G) > kSharedMaxSlots)
    return GDNTREE_ERR_UNSUPPORTED;
  if (gdntree_status st = device_ok(); st != GDNTREE_OK) return st;
  const BuildParams bp{lat_logp, lat_tok, root_tok, P, K, N, out, positions};
  if (launch_build_shared(bp, B, G, stream) != hipSuccess) return GDNTREE_ERR_DEVICE;
  return GDNTREE_OK;
}

GDNTREE_EXPORT gdntree_status gdntree_verify(gdntree_tree tree, int B, int N, int L, int H, int dk,
                                             int dv, gdntree_dtype in_dtype, const void *q,
                                             const void *k, const void *v, const void *alpha,
                                             const void *beta, const float *state,
                                             gdntree_dtype out_dtype, void *o, hipStream_t stream) {
  if (!tree.parent || !tree.anc || !tree.n_nodes || !q || !k || !v || !alpha || !beta || !state || !o)
    return GDNTREE_ERR_ARG;
  if (B <= 0 || N <= 0 || L <= 0 || H <= 0) return GDNTREE_ERR_ARG;
  if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return GDNTREE_ERR_ARG;
  if (gdntree_status st = head_dims(dk, dv); st != GDNTREE_OK) return st;
  if (N > kMaxN || !grid_fits((long long)L * B * H)) return GDNTREE_ERR_UNSUPPORTED;
  if (gdntree_status st = device_ok(); st != GDNTREE_OK) return st;
  VerifyParams p;
  p.parent = tree.parent;
  p.anc = reinterpret_cast<const unsigned long long *>(tree.anc);
  p.n_nodes = tree.n_nodes;
  p.q = q; p.k = k; p.v = v; p.alpha = alpha; p.beta = beta;
  p.state = state;
  p.o = o;
  p.B = B; p.R = N + 1; p.L = L; p.H = H; p.D = dk;
  p.in_bf16 = in_dtype == GDNTREE_BF16;
  p.out_bf16 = out_dtype == GDNTREE_BF16;
  if (launch_verify(p, stream) != hipSuccess) return GDNTREE_ERR_DEVICE;
  return GDNTREE_OK;
}

GDNTREE_EXPORT gdntree_status gdntree_accept_commit(gdntree_tree tree, int B, int N, int P,
                                                    const int32_t *target_argmax, int L, int H,
                                                    int dk, int dv, gdntree_dtype in_dtype,
                                                    const void *k, const void *v, const void *alpha,
                                                    const void *beta, float *state, int32_t *acc_len,
                                                    int32_t *acc_tok, int32_t *acc_node,
                                                    hipStream_t stream) {
  if (!tree.parent || !tree.token || !tree.n_nodes || !target_argmax || !k || !v || !alpha ||
      !beta || !state || !acc_len || !acc_tok || !acc_node)
    return GDNTREE_ERR_ARG;
  if (B <= 0 || N <= 0 || P <= 0 || L <= 0 || H <= 0) return GDNTREE_ERR_ARG;
  if (!dtype_ok(in_dtype)) return GDNTREE_ERR_ARG;
  if (gdntree_status st = head_dims(dk, dv); st != GDNTREE_OK) return st;
  if (N > kMaxN || P > kMaxP || !grid_fits((long long)L * B * H)) return GDNTREE_ERR_UNSUPPORTED;
  if (gdntree_status st = device_ok(); st != GDNTREE_OK) return st;
  CommitParams p;
  p.parent = tree.parent; p.token = tree.token; p.n_nodes = tree.n_nodes; p.target = target_argmax;
  p.k = k; p.v = v; p.alpha = alpha; p.beta = beta;
  p.state = state;
  p.acc_len = acc_len; p.acc_tok = acc_tok; p.acc_node = acc_node;
  p.B = B; p.R = N + 1; p.P = P; p.L = L; p.H = H; p.D = dk;
  p.in_bf16 = in_dtype == GDNTREE_BF16;
  if (launch_accept_commit(p, stream) != hipSuccess) return GDNTREE_ERR_DEVICE;
  return GDNTREE_OK;
}

GDNTREE_EXPORT gdntree_status gdntree_accept(gdntree_tree tree, int B, int N, int P,
                                             const int32_t *target_argmax, int32_t *acc_len,
                                             int32_t *acc_tok, int32_t *acc_node, hipStream_t stream) {
  if (!tree.parent || !tree.token || !tree.n_nodes || !target_argmax || !acc_len || !acc_tok || !acc_node)
    return GDNTREE_ERR_ARG;
  if (B <= 0 || N <= 0 || P <= 0) return GDNTREE_ERR_ARG;
  if (N > kMaxN || P > kMaxP || !grid_fits(B)) return GDNTREE_ERR_UNSUPPORTED;
  if (gdntree_status st = device_ok(); st != GDNTREE_OK) return st;
  CommitParams p{};
  p.parent = tree.parent; p.token = tree.token; p.n_nodes = tree.n_nodes; p.target = target_argmax;
  p.acc_len = acc_len; p.acc_tok = acc_tok; p.acc_node = acc_node;
  p.B = B; p.R = N + 1; p.P = P; p.L = 1; p.H = 1; p.D = 128;
  if (launch_accept(p, stream) != hipSuccess) return GDNTREE_ERR_DEVICE;
  return GDNTREE_OK;
}

GDNTREE_EXPORT gdntree_status gdntree_commit(gdntree_tree tree, int B, int N, int P,
                                             const int32_t *acc_len, const int32_t *acc_node, int L,
                                             int H, int dk, int dv, gdntree_dtype in_dtype,
                                             const void *k, const void *v, const void *alpha,
                                             const void *beta, float *state, hipStream_t stream) {
  if (!tree.parent || !tree.n_nodes || !acc_len || !acc_node || !k || !v || !alpha || !beta || !state)
    return GDNTREE_ERR_ARG;
  if (B <= 0 || N <= 0 || P <= 0 || L <= 0 || H <= 0) return GDNTREE_ERR_ARG;
  if (!dtype_ok(in_dtype)) return GDNTREE_ERR_ARG;
  if (gdntree_status st = head_dims(dk, dv); st != GDNTREE_OK) return st;
  if (N > kMaxN || P > kMaxP || !grid_fits((long long)L * B * H)) return GDNTREE_ERR_UNSUPPORTED;
  if (gdntree_status st = device_ok(); st != GDNTREE_OK) return st;
  CommitParams p{};
  p.parent = tree.parent; p.n_nodes = tree.n_nodes;
  p.k = k; p.v = v; p.alpha = alpha; p.beta = beta;
  p.state = state;
  // read only by this kernel (the acceptance outputs of a previous call)
  p.acc_len = const_cast<int32_t *>(acc_len); p.acc_node = const_cast<int32_t *>(acc_node);
  p.B = B; p.R = N + 1; p.P = P; p.L = L; p.H = H; p.D = dk;
  p.in_bf16 = in_dtype == GDNTREE_BF16;
  if (launch_commit(p, stream) != hipSuccess) return GDNTREE_ERR_DEVICE;
  return GDNTREE_OK;
}

GDNTREE_EXPORT gdntree_status gdntree_commit_build(
    gdntree_tree tree, int B, int N, int P, const int32_t *acc_len, const int32_t *acc_node, int L,
    int H, int dk, int dv, gdntree_dtype in_dtype, const void *k, const void *v, const void *alpha,
    const void *beta, float *state, const float *next_lat_logp, const int32_t *next_lat_tok,
    const int32_t *next_root_tok, int next_B, int next_P, int next_K, int next_N,
    gdntree_tree next_tree, hipStream_t stream) {
  if (!tree.parent || !tree.n_nodes || !acc_len || !acc_node || !k || !v || !alpha || !beta || !state)
    return GDNTREE_ERR_ARG;
  if (!next_lat_logp || !next_lat_tok || !next_root_tok || !next_tree.parent || !next_tree.depth ||
      !next_tree.rank || !next_tree.token || !next_tree.score || !next_tree.anc || !next_tree.n_nodes)
    return GDNTREE_ERR_ARG;
  // the commit reads the current tree while the build writes the next one
  if (next_tree.parent == tree.parent || next_tree.n_nodes == tree.n_nodes) return GDNTREE_ERR_ARG;
  if (B <= 0 || N <= 0 || P <= 0 || L <= 0 || H <= 0) return GDNTREE_ERR_ARG;
  if (next_B <= 0 || next_P <= 0 || next_K <= 0 || next_N <= 0) return GDNTREE_ERR_ARG;
  if (!dtype_ok(in_dtype)) return GDNTREE_ERR_ARG;
  if (gdntree_status st = head_dims(dk, dv); st != GDNTREE_OK) return st;
  if (N > kMaxN || P > kMaxP || next_P > kMaxP || next_K > kMaxK || next_N > kMaxN ||
      !grid_fits((long long)L * B * H + next_B))
    return GDNTREE_ERR_UNSUPPORTED;
  if (gdntree_status st = device_ok(); st != GDNTREE_OK) return st;
  CommitParams p{};
  p.parent = tree.parent; p.n_nodes = tree.n_nodes;
  p.k = k; p.v = v; p.alpha = alpha; p.beta = beta;
  p.state = state;
  p.acc_len = const_cast<int32_t *>(acc_len); p.acc_node = const_cast<int32_t *>(acc_node);
  p.B = B; p.R = N + 1; p.P = P; p.L = L; p.H = H; p.D = dk;
  p.in_bf16 = in_dtype == GDNTREE_BF16;
  const BuildParams bp{next_lat_logp, next_lat_tok, next_root_tok, next_P, next_K, next_N, next_tree, nullptr};
  if (launch_commit_build(p, bp, next_B, stream) != hipSuccess) return GDNTREE_ERR_DEVICE;
  return GDNTREE_OK;
}

namespace {

// The fused acceptance + commit + next build, optionally followed by the cut of the next
// trees to a batch budget of next_G draft nodes (next_G < 0: no budget).
gdntree_status accept_commit_build_impl(
    gdntree_tree tree, int B, int N, int P, const int32_t *target_argmax, int L, int H, int dk,
    int dv, gdntree_dtype in_dtype, const void *k, const void *v, const void *alpha,
    const void *beta, float *state, int32_t *acc_len, int32_t *acc_tok, int32_t *acc_node,
    const float *next_lat_logp, const int32_t *next_lat_tok, const int32_t *next_root_tok,
    const int32_t *next_positions, int next_B, int next_P, int next_K, int next_N, int next_G,
    gdntree_tree next_tree, hipStream_t stream) {
  if (!tree.parent || !tree.token || !tree.n_nodes || !target_argmax || !k || !v || !alpha ||
      !beta || !state || !acc_len || !acc_tok || !acc_node)
    return GDNTREE_ERR_ARG;
  if (!next_lat_logp || !next_lat_tok || !next_root_tok || !next_tree.parent || !next_tree.depth ||
      !next_tree.rank || !next_tree.token || !next_tree.score || !next_tree.anc || !next_tree.n_nodes)
    return GDNTREE_ERR_ARG;
  // the acceptance and commit read the current tree while the build writes the next one
  if (next_tree.parent == tree.parent || next_tree.n_nodes == tree.n_nodes || next_tree.token == tree.token)
    return GDNTREE_ERR_ARG;
  if (B <= 0 || N <= 0 || P <= 0 || L <= 0 || H <= 0) return GDNTREE_ERR_ARG;
  if (next_B <= 0 || next_P <= 0 || next_K <= 0 || next_N <= 0) return GDNTREE_ERR_ARG;
  if (!dtype_ok(in_dtype)) return GDNTREE_ERR_ARG;
  if (gdntree_status st = head_dims(dk, dv); st != GDNTREE_OK) return st;
  if (N > kMaxN || P > kMaxP || next_P > kMaxP || next_K > kMaxK || next_N > kMaxN ||
      !grid_fits((long long)L * B * H + (next_B > B ? next_B : B)))
    return GDNTREE_ERR_UNSUPPORTED;
  if (next_G >= 0) {
    if (next_B > kSharedMaxB) return GDNTREE_ERR_UNSUPPORTED;
    if (next_G > 0 && (long long)next_G < (long long)next_B * next_N &&
        (long long)shared_budget_lists(next_B) * (next_N < next_G ? next_N : next_G) > kSharedMaxSlots)
      return GDNTREE_ERR_UNSUPPORTED;
  }
  if (gdntree_status st = device_ok(); st != GDNTREE_OK) return st;
  CommitParams p{};
  p.parent = tree.parent; p.token = tree.token; p.n_nodes = tree.n_nodes; p.target = target_argmax;
  p.k = k; p.v = v; p.alpha = alpha; p.beta = beta;
  p.state = state;
  p.acc_len = acc_len; p.acc_tok = acc_tok; p.acc_node = acc_node;
  p.B = B; p.R = N + 1; p.P = P; p.L = L; p.H = H; p.D = dk;
  p.in_bf16 = in_dtype == GDNTREE_BF16;
  const BuildParams bp{next_lat_logp, next_lat_tok, next_root_tok, next_P, next_K, next_N, next_tree, next_positions};
  if (launch_accept_commit_build(p, bp, next_B, stream) != hipSuccess) return GDNTREE_ERR_DEVICE;
  if (next_G >= 0 && launch_budget_cut(next_tree, next_B, next_N, next_G, stream) != hipSuccess)
    return GDNTREE_ERR_DEVICE;
  return GDNTREE_OK;
}

}  // namespace

GDNTREE_EXPORT gdntree_status gdntree_accept_commit_build(
    gdntree_tree tree, int B, int N, int P, const int32_t *target_argmax, int L, int H, int dk,
    int dv, gdntree_dtype in_dtype, const void *k, const void *v, const void *alpha,
    const void *beta, float *state, int32_t *acc_len, int32_t *acc_tok, int32_t *acc_node,
    const float *next_lat_logp, const int32_t *next_lat_tok, const int32_t *next_root_tok,
    int next_B, int next_P, int next_K, int next_N, gdntree_tree next_tree, hipStream_t stream) {
  return accept_commit_build_impl(tree, B, N, P, target_argmax, L, H, dk, dv, in_dtype, k, v, alpha, beta, state,
                                  acc_len, acc_tok, acc_node, next_lat_logp, next_lat_tok, next_root_tok, nullptr,
                                  next_B, next_P, next_K, next_N, -1, next_tree, stream);
}

GDNTREE_EXPORT gdntree_status gdntree_accept_commit_build_shared(
    gdntree_tree tree, int B, int N, int P, const int32_t *target_argmax, int L, int H, int dk,
    int dv, gdntree_dtype in_dtype, const void *k, const void *v, const void *alpha,
    const void *beta, float *state, int32_t *acc_len, int32_t *acc_tok, int32_t *acc_node,
    const float *next_lat_logp, const int32_t *next_lat_tok, const int32_t *next_root_tok,
    const int32_t *next_positions, int next_B, int next_P, int next_K, int next_N, int next_G,
    gdntree_tree next_tree, hipStream_t stream) {
  if (next_G < 0) return GDNTREE_ERR_ARG;
  return accept_commit_build_impl(tree, B, N, P, target_argmax, L, H, dk, dv, in_dtype, k, v, alpha, beta, state,
                                  acc_len, acc_tok, acc_node, next_lat_logp, next_lat_tok, next_root_tok,
                                  next_positions, next_B, next_P, next_K, next_N, next_G, next_tree, stream);
}

GDNTREE_EXPORT gdntree_status gdntree_accept_build(gdntree_tree tree, int B, int N, int P,
                                                   const int32_t *target_argmax, int32_t *acc_len,
                                                   int32_t *acc_tok, int32_t *acc_node,
                                                   const float *next_lat_logp, const int32_t *next_lat_tok,
                                                   const int32_t *next_root_tok, int next_B, int next_P,
                                                   int next_K, int next_N, gdntree_tree next_tree,
                                                   hipStream_t stream) {
  if (!tree.parent || !tree.token || !tree.n_nodes || !target_argmax || !acc_len || !acc_tok || !acc_node)
    return GDNTREE_ERR_ARG;
  if (!next_lat_logp || !next_lat_tok || !next_root_tok || !next_tree.parent || !next_tree.depth ||
      !next_tree.rank || !next_tree.token || !next_tree.score || !next_tree.anc || !next_tree.n_nodes)
    return GDNTREE_ERR_ARG;
  // the acceptance reads the current tree while the build writes the next one
  if (next_tree.parent == tree.parent || next_tree.n_nodes == tree.n_nodes || next_tree.token == tree.token)
    return GDNTREE_ERR_ARG;
  if (B <= 0 || N <= 0 || P <= 0 || next_B <= 0 || next_P <= 0 || next_K <= 0 || next_N <= 0)
    return GDNTREE_ERR_ARG;
  if (N > kMaxN || P > kMaxP || next_P > kMaxP || next_K > kMaxK || next_N > kMaxN ||
      !grid_fits(next_B > B ? next_B : B))
    return GDNTREE_ERR_UNSUPPORTED;
  if (gdntree_status st = device_ok(); st != GDNTREE_OK) return st;
  CommitParams p{};  // no commit workgroups (L = 0)
  p.parent = tree.parent; p.token = tree.token; p.n_nodes = tree.n_nodes; p.target = target_argmax;
  p.acc_len = acc_len; p.acc_tok = acc_tok; p.acc_node = acc_node;
  p.B = B; p.R = N + 1; p.P = P; p.L = 0; p.H = 1; p.D = 128; p.in_bf16 = 1;
  const BuildParams bp{next_lat_logp, next_lat_tok, next_root_tok, next_P, next_K, next_N, next_tree, nullptr};
  if (launch_accept_commit_build(p, bp, next_B, stream) != hipSuccess) return GDNTREE_ERR_DEVICE;
  return GDNTREE_OK;
}

GDNTREE_EXPORT gdntree_status gdntree_accept_commit_verify(
    gdntree_tree prev_tree, int prev_N, int prev_P, const int32_t *prev_target_argmax,
    const void *prev_k, const void *prev_v, const void *prev_alpha, const void *prev_beta,
    int32_t *acc_len, int32_t *acc_tok, int32_t *acc_node, gdntree_tree tree, int B, int N, int L,
    int H, int dk, int dv, gdntree_dtype in_dtype, const void *q, const void *k, const void *v,
    const void *alpha, const void *beta, float *state, gdntree_dtype out_dtype, void *o,
    hipStream_t stream) {
  if (!prev_tree.parent || !prev_tree.token || !prev_tree.n_nodes || !prev_target_argmax || !prev_k ||
      !prev_v || !prev_alpha || !prev_beta)
    return GDNTREE_ERR_ARG;
  if (!tree.parent || !tree.anc || !tree.n_nodes || !q || !k || !v || !alpha || !beta || !state || !o)
    return GDNTREE_ERR_ARG;
  const int nacc = (acc_len != nullptr) + (acc_tok != nullptr) + (acc_node != nullptr);
  if (nacc != 0 && nacc != 3) return GDNTREE_ERR_ARG;  // all three acceptance outputs, or none
  if (B <= 0 || N <= 0 || L <= 0 || H <= 0 || prev_N <= 0 || prev_P <= 0) return GDNTREE_ERR_ARG;
  if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return GDNTREE_ERR_ARG;
  if (gdntree_status st = head_dims(dk, dv); st != GDNTREE_OK) return st;
  if (N > kMaxN || prev_N > kMaxN || prev_P > kMaxP || !grid_fits((long long)L * B * H))
    return GDNTREE_ERR_UNSUPPORTED;
  if (gdntree_status st = device_ok(); st != GDNTREE_OK) return st;
  VerifyParams p;
  p.parent = tree.parent;
  p.anc = reinterpret_cast<const unsigned long long *>(tree.anc);
  p.n_nodes = tree.n_nodes;
  p.q = q; p.k = k; p.v = v; p.alpha = alpha; p.beta = beta;
  p.state = state;
  p.o = o;
  p.B = B; p.R = N + 1; p.L = L; p.H = H; p.D = dk;
  p.in_bf16 = in_dtype == GDNTREE_BF16;
  p.out_bf16 = out_dtype == GDNTREE_BF16;
  p.pv_parent = prev_tree.parent; p.pv_token = prev_tree.token; p.pv_n_nodes = prev_tree.n_nodes;
  p.pv_target = prev_target_argmax;
  p.pv_k = prev_k; p.pv_v = prev_v; p.pv_alpha = prev_alpha; p.pv_beta = prev_beta;
  p.acc_len = acc_len; p.acc_tok = acc_tok; p.acc_node = acc_node;
  p.pv_R = prev_N + 1; p.pv_P = prev_P;
  if (launch_verify(p, stream) != hipSuccess) return GDNTREE_ERR_DEVICE;
  return GDNTREE_OK;
}

GDNTREE_EXPORT const char *gdntree_status_str(gdntree_status status) {
  switch (status) {
    case GDNTREE_OK: return "ok";
    case GDNTREE_ERR_ARG: return "invalid argument (null pointer, non-positive size or unknown dtype)";
    case GDNTREE_ERR_UNSUPPORTED: return "unsupported size (N<=64, P<=16, K<=64, d_k=d_v in {64,128})";
    case GDNTREE_ERR_DEVICE: return "no usable HIP device or kernel launch failed";
    default: return "unknown status";
  }
}
