/*
 * gdntree.h - C ABI of the gfx950 library for lossless draft-tree verification of
 * speculative decoding against a hybrid Gated-DeltaNet (GDN) target.
 *
 * One decode step is three calls on one stream:
 *   gdntree_build          best-first draft tree from the drafter's top-K lattice
 *   gdntree_verify         gated-delta-rule outputs of every tree node, per GDN layer
 *   gdntree_accept_commit  greedy acceptance of the longest matching root path plus a
 *                          bonus token, then the accepted-path state commit
 * gdntree_build_shared builds the trees of a whole batch under one shared node budget, and
 * gdntree_accept_commit_build_shared fuses that build into the end of the previous step.
 * gdntree_accept_commit also comes as two calls, gdntree_accept then gdntree_commit, and
 * gdntree_commit_build / gdntree_accept_commit_build run a commit (with or without the
 * acceptance) together with the next step's tree build in one launch.  Alternatively the
 * commit is deferred into the next step's verify: gdntree_accept_build (acceptance + next
 * build), then gdntree_accept_commit_verify (acceptance + commit + verify of the next tree).  For a drafter whose
 * candidate scores depend on the previous token (a Markov head), gdntree_markov_edges forms
 * the parent-conditioned edge log-probs and gdntree_build_cond builds the tree over them.
 *
 * Sources: the SpecPilot paper summary (paper.rainbus.top, "SpecPilot: Autonomous
 * Algorithm Discovery and Systems Optimization for Speculative Decoding"), sections
 * Prerequisites > speculative decoding, > parallel drafter, > draft-tree verification,
 * > hybrid recurrent architecture, and Technical novelty.
 *
 * Conventions shared by every call
 *  - Every array argument is a DEVICE pointer to memory the caller owns.  The library never
 *    allocates, frees or synchronises; it validates arguments on the host, enqueues its
 *    kernels on `stream` (NULL = the default stream) and returns.
 *  - Layouts are dense row-major with the shapes given; no strides.
 *  - On any error nothing is enqueued and no output is touched (except ERR_DEVICE after a
 *    failed launch, when the stream state is the runtime's).  No C++ exception crosses the
 *    ABI.  The library holds no global state and is safe to call from several threads;
 *    calls are ordered only through their streams.
 *  - Slot t of a request's tree holds node t; slot 0 is the root (the pending last token,
 *    processed first from the committed state), draft slots 1..N follow in insertion order
 *    and every parent index is smaller than its child's.  Slots >= n_nodes[b] are never
 *    read and never written.
 *  - Limits: 1 <= N <= 64 draft nodes, 1 <= P <= 16 positions (so tree depth <= 16),
 *    1 <= K <= 64 candidates, d_k = d_v in {64, 128}.
 */
#ifndef GDNTREE_H
#define GDNTREE_H

#include <stdint.h>

#include <hip/hip_runtime_api.h> /* hipStream_t */

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GDNTREE_OK = 0,
  GDNTREE_ERR_ARG = 1,          /* null pointer, non-positive size, unknown dtype          */
  GDNTREE_ERR_UNSUPPORTED = 2,  /* a size beyond the limits above, or d_k != d_v            */
  GDNTREE_ERR_DEVICE = 3        /* no usable HIP device, or a kernel launch failed          */
} gdntree_status;

typedef enum { GDNTREE_F32 = 0, GDNTREE_BF16 = 1 } gdntree_dtype;

/* One best-first tree per request, N+1 slots each ([B][N+1] arrays). */
typedef struct {
  int32_t *parent;   /* parent slot; -1 for the root                                       */
  int32_t *depth;    /* root 0; a draft at lattice position p has depth p+1                */
  int32_t *rank;     /* candidate rank at position depth-1; -1 for the root                */
  int32_t *token;    /* token id; the root holds root_tok[b]                               */
  double *score;     /* cumulative path log-prob, summed root to leaf in fp64; root 0.0   */
  uint64_t *anc;     /* bit j-1 set iff draft slot j is an ancestor-or-self; root 0        */
                     /* (the attention tree mask of the target's attention layers)         */
  int32_t *n_nodes;  /* [B] slots in use, root included (N+1 unless the trie ran out)      */
} gdntree_tree;

/*
 * gdntree_build - best-first (DDTree-style) tree over the drafter lattice.
 *
 * Starting from the root, repeatedly inserts the not-yet-inserted lattice child with the
 * largest cumulative path log-prob score(parent) + lat_logp[b][depth(parent)][rank] until
 * N draft nodes exist or the trie (positions 0..P-1) is exhausted.  Ties go to the smaller
 * parent slot, then the smaller rank.  Scores are fp64 sums of the fp32 log-probs, added
 * root to leaf, so topology and scores are bit-reproducible.  (SpecPilot summary,
 * Prerequisites > draft-tree verification: nodes added greedily by path log-prob up to N;
 * Technical novelty: edges scored by log p(child | parent), trees wider than the block.)
 *
 *   lat_logp  f32 [B][P][K]  candidate log-probs per position, NON-INCREASING along K
 *                            (a sorted top-K); an unsorted row yields a valid tree that
 *                            may differ from the best-first one.  Must not hold NaN; -inf
 *                            is allowed (such a candidate, and its subtree, comes after
 *                            every finite one, and still counts toward N).
 *   lat_tok   i32 [B][P][K]  candidate token ids (distinct within a position)
 *   root_tok  i32 [B]        the pending last token of each request
 *   out                      every field written for slots < n_nodes[b]
 */
gdntree_status gdntree_build(const float *lat_logp, const int32_t *lat_tok,
                             const int32_t *root_tok, int B, int P, int K, int N,
                             gdntree_tree out, hipStream_t stream);

/*
 * gdntree_build_shared - best-first trees for a whole batch under one shared node budget.
 *
 * One best-first pass over the union of every request's frontier: it inserts the batch's
 * candidate with the largest cumulative path log-prob until the batch holds G draft nodes
 * (roots not counted) or no candidate is left.  A request holding N draft nodes offers no
 * more, and request b takes children only from its first positions[b] lattice positions.
 * Ties go to the smaller request index, then the smaller parent slot, then the smaller
 * rank.  Each request's tree is then exactly the prefix of its own gdntree_build tree (over
 * its positions) that the budget leaves it.  (SpecPilot summary, Technical novelty,
 * batching: a node budget shared by the batch, draft positions chosen per request.)
 *
 *   lat_logp, lat_tok, root_tok  as for gdntree_build
 *   positions i32 [B] or NULL    draft positions per request, clipped to [0, P] (0: the
 *                                request gets its root only); NULL: P for every request
 *   G                            the batch's draft-node budget, G >= 0 (0: roots only)
 *   out                          every field written for slots < n_nodes[b]; slots at or
 *                                past n_nodes[b] may hold nodes the budget cut off
 * Limits: B <= 1024 and, when 0 < G < B * N, B' * min(N, G) <= 4096 with B' = B rounded up
 * to a power of two (else ERR_UNSUPPORTED).  lat_logp must hold log-probabilities (<= 0), so
 * that a child never outscores its parent.  Two kernels: the per-request builds, then (when
 * G < B * N) one workgroup that merges the requests' score lists under (score desc, request,
 * slot), keeping the first G keys, and cuts every n_nodes[b] to its slots among them.
 */
gdntree_status gdntree_build_shared(const float *lat_logp, const int32_t *lat_tok,
                                    const int32_t *root_tok, const int32_t *positions, int B,
                                    int P, int K, int N, int G, gdntree_tree out, hipStream_t stream);

/*
 * gdntree_markov_edges - parent-conditioned edge log-probs of a DSpark-style Markov head.
 *
 * The head scores candidate y at position s as l_s(y) = bases(y) + <W1[x_{s-1}], W2[y]>,
 * x_{s-1} the previous token (SpecPilot summary, Prerequisites > parallel drafter).  A
 * child's previous token is its parent's: the root token at position 0, else the parent's
 * candidate at position s-1.  A position's candidates stay its K lattice tokens; only their
 * scores depend on the parent.
 *
 *   bases     f32 [B][P][K]      base logits of the lattice candidates
 *   lat_tok   i32 [B][P][K]      candidate token ids (in [0, V))
 *   root_tok  i32 [B]            the pending last token of each request (in [0, V))
 *   W1, W2    [V][R], w_dtype    previous-token and candidate embeddings (f32 or bf16)
 *   edge_logp f32 [B][P][K][K]   out: [b][s][pr][r] = l_s(candidate r | the previous token of
 *                                row pr) minus the log-sum-exp of l_s over the K candidates of
 *                                position s; row pr's previous token is candidate pr of
 *                                position s-1 (s >= 1) or the root token (s = 0, every row)
 * Arithmetic in fp32 (the dot products in order over R, a max-shifted log-sum-exp).  A token
 * id outside [0, V) reads an all-zero embedding row.  Limits: P <= 16, K <= 64, R <= 64,
 * V * R * (element size) < 2^31 (else ERR_UNSUPPORTED).
 */
gdntree_status gdntree_markov_edges(const float *bases, const int32_t *lat_tok, const int32_t *root_tok,
                                    const void *W1, const void *W2, gdntree_dtype w_dtype, int B, int P,
                                    int K, int V, int R, float *edge_logp, hipStream_t stream);

/*
 * gdntree_build_cond - best-first draft tree over parent-conditioned edge log-probs.
 *
 * As gdntree_build, except that the log-prob of child rank r of node p is
 * edge_logp[b][depth(p)][pr][r] with pr = rank(p), the parent's own candidate at its position
 * (pr = 0 for the root's children): edges scored by log p(child | parent) (SpecPilot summary,
 * Technical novelty).  Scores are fp64 sums of these fp32 log-probs root to leaf; ties go to
 * the smaller parent slot, then the smaller rank.  The rows need not be sorted: each row is
 * sorted once and a node offers its children in that order, which is the tie rule's order
 * whenever distinct log-probs of a row give distinct fp64 sums with the node's score (rows of
 * log-probabilities do for every score above -1e8); a node scored -inf offers its children,
 * all tied at -inf, in rank order.
 *
 *   edge_logp f32 [B][P][K][K]   e.g. from gdntree_markov_edges; no NaN (-inf allowed)
 *   lat_tok, root_tok, out       as for gdntree_build
 * Limits: P <= 16, K <= 16, N <= 64 (else ERR_UNSUPPORTED).
 */
gdntree_status gdntree_build_cond(const float *edge_logp, const int32_t *lat_tok, const int32_t *root_tok,
                                  int B, int P, int K, int N, gdntree_tree out, hipStream_t stream);

/*
 * gdntree_verify - per-node gated delta rule over the tree, one or more layers.
 *
 * For every layer l, request b, head h and slot t < n_nodes[b], with S_p the state of
 * t's parent (the committed state h0 = state[l][b][h] for the root):
 *     S_t = alpha_t (I - beta_t k_t k_t^T) S_p + beta_t k_t v_t^T,    o_t = S_t^T q_t
 * (SpecPilot summary, Prerequisites > hybrid recurrent architecture).  Node states are
 * derived along root paths from h0 and never written to memory (no per-node snapshots);
 * only o is written.  No 1/sqrt(d_k) scale is applied.  Arithmetic: the products of the
 * state with the q and k rows are fp32-exact on the matrix cores (each fp32 state entry is
 * split into three bf16 parts that hold its 24-bit significand exactly; bf16 rows enter as
 * they are, fp32 rows are split likewise), accumulated in fp32; the tree terms (Gram entries
 * of ancestor pairs, the per-node path solves, the gates) and the final sums are fp32.
 *
 * Reads tree.parent, tree.anc and tree.n_nodes only (the ancestor bitmask gives each
 * node's depth and ancestors).  A request whose tree is inconsistent (parent[t] >= t,
 * anc[t] != anc[parent[t]] | bit t-1, anc[0] != 0, or depth > 16) gets NaN outputs in all
 * of its slots < n_nodes; a request with n_nodes outside [1, N+1] gets no output at all.
 *
 *   q, k      in_dtype [L][B][N+1][H][d_k]
 *   v         in_dtype [L][B][N+1][H][d_v]
 *   alpha     in_dtype [L][B][N+1][H]   decay gate in (0, 1]
 *   beta      in_dtype [L][B][N+1][H]   write strength
 *   state     f32 [L][B][H][d_k][d_v]   committed state S (row i = key channel, column j =
 *             value channel), read only
 *   o         out_dtype [L][B][N+1][H][d_v]  written for slots < n_nodes[b]
 */
gdntree_status gdntree_verify(gdntree_tree tree, int B, int N, int L, int H, int dk, int dv,
                              gdntree_dtype in_dtype, const void *q, const void *k,
                              const void *v, const void *alpha, const void *beta,
                              const float *state, gdntree_dtype out_dtype, void *o,
                              hipStream_t stream);

/*
 * gdntree_accept_commit - greedy acceptance plus bonus, then the accepted-path commit.
 *
 * Acceptance (SpecPilot summary, Prerequisites > speculative decoding and > draft-tree
 * verification): u <- root; while some child c of u has token[c] == target_argmax[u]
 * (the smallest such slot), u <- c.  tau = accepted drafts + 1, at most P+1.  The emitted
 * tokens are the accepted drafts' tokens followed by the bonus target_argmax[u].
 * Commit: for every layer and head, state[l][b][h] <- the state of node u, recomputed in
 * fp32 from the committed state along root -> u with the gated delta rule and written in
 * place (same [d_k][d_v] layout as gdntree_verify).
 *
 *   target_argmax  i32 [B][N+1]  the target's argmax after each slot's node
 *   k, v, alpha, beta            as for gdntree_verify (rows of the accepted slots are read)
 *   state          f32 [L][B][H][d_k][d_v], updated in place
 *   acc_len        i32 [B]       tau
 *   acc_tok        i32 [B][P+1]  accepted draft tokens then the bonus; padded with -1
 *   acc_node       i32 [B][P+1]  root slot 0 then the accepted slots; padded with -1
 * Reads tree.parent, tree.token and tree.n_nodes.
 */
gdntree_status gdntree_accept_commit(gdntree_tree tree, int B, int N, int P,
                                     const int32_t *target_argmax, int L, int H, int dk,
                                     int dv, gdntree_dtype in_dtype, const void *k,
                                     const void *v, const void *alpha, const void *beta,
                                     float *state, int32_t *acc_len, int32_t *acc_tok,
                                     int32_t *acc_node, hipStream_t stream);

/*
 * gdntree_accept - the acceptance half of gdntree_accept_commit on its own (one wave per
 * request): the same acc_len, acc_tok and acc_node, and no state is touched.  With
 * gdntree_commit it splits a step's end in two, so that work that needs only the accepted
 * tokens (the next draft and tree build) can start on another stream while the states are
 * being committed.  Reads tree.parent, tree.token, tree.n_nodes and target_argmax; a request
 * with n_nodes outside [1, N+1] gets no output.
 */
gdntree_status gdntree_accept(gdntree_tree tree, int B, int N, int P,
                              const int32_t *target_argmax, int32_t *acc_len, int32_t *acc_tok,
                              int32_t *acc_node, hipStream_t stream);

/*
 * gdntree_commit - the commit half of gdntree_accept_commit for an accepted path given by a
 * previous gdntree_accept on the same tree (same sources): for every layer and head,
 * state[l][b][h] <- the state of node acc_node[b][acc_len[b] - 1], recomputed in fp32 from
 * the committed state along acc_node[b][0..acc_len[b]) and written in place.
 *
 *   acc_len   i32 [B]        read only
 *   acc_node  i32 [B][P+1]   read only
 *   the rest as for gdntree_accept_commit.
 * A request whose path is not a root path of its tree (acc_len outside [1, P+1], a first
 * slot other than 0, a slot outside [1, n_nodes) or whose parent is not the previous slot)
 * or whose n_nodes lies outside [1, N+1] keeps its state unchanged.  Reads tree.parent and
 * tree.n_nodes.
 */
gdntree_status gdntree_commit(gdntree_tree tree, int B, int N, int P, const int32_t *acc_len,
                              const int32_t *acc_node, int L, int H, int dk, int dv,
                              gdntree_dtype in_dtype, const void *k, const void *v,
                              const void *alpha, const void *beta, float *state, hipStream_t stream);

/*
 * gdntree_commit_build - gdntree_commit for this step's batch and gdntree_build for the next
 * step's lattices in ONE launch (same sources as both).  The commit is bound by HBM traffic
 * and the build is a latency-bound chain per request, so in one launch the build runs
 * beside the commit instead of after it; results are exactly those of the two calls.
 * Enqueue it after this step's gdntree_accept: the next draft, and so the next lattice,
 * needs the accepted tokens.
 *
 *   tree ... state         as for gdntree_commit (this step)
 *   next_lat_logp ... next_N, next_tree   as for gdntree_build (the next step)
 * next_tree must not share memory with tree (the commit reads tree while the build writes
 * next_tree); equal parent or n_nodes pointers give ERR_ARG.  Every check of the two calls
 * applies; on any error nothing is enqueued.
 */
gdntree_status gdntree_commit_build(gdntree_tree tree, int B, int N, int P,
                                    const int32_t *acc_len, const int32_t *acc_node, int L,
                                    int H, int dk, int dv, gdntree_dtype in_dtype,
                                    const void *k, const void *v, const void *alpha,
                                    const void *beta, float *state,
                                    const float *next_lat_logp, const int32_t *next_lat_tok,
                                    const int32_t *next_root_tok, int next_B, int next_P,
                                    int next_K, int next_N, gdntree_tree next_tree,
                                    hipStream_t stream);

/*
 * gdntree_accept_commit_build - gdntree_accept_commit for this step and gdntree_build for
 * the next step's lattices in ONE launch (same sources as both).  Request b's next tree is
 * built by the workgroup that has just walked request b's acceptance, so each next build
 * starts after its own request's acceptance, as the next draft requires; the commit runs
 * beside the builds.  Results are exactly those of gdntree_accept_commit followed by
 * gdntree_build.
 *
 *   tree ... acc_node      as for gdntree_accept_commit (this step)
 *   next_lat_logp ... next_N, next_tree   as for gdntree_build (the next step)
 * next_tree must not share memory with tree; equal parent, token or n_nodes pointers give
 * ERR_ARG.  Every check of the two calls applies; on any error nothing is enqueued.
 */
gdntree_status gdntree_accept_commit_build(gdntree_tree tree, int B, int N, int P,
                                           const int32_t *target_argmax, int L, int H, int dk,
                                           int dv, gdntree_dtype in_dtype, const void *k,
                                           const void *v, const void *alpha, const void *beta,
                                           float *state, int32_t *acc_len, int32_t *acc_tok,
                                           int32_t *acc_node, const float *next_lat_logp,
                                           const int32_t *next_lat_tok,
                                           const int32_t *next_root_tok, int next_B, int next_P,
                                           int next_K, int next_N, gdntree_tree next_tree,
                                           hipStream_t stream);

/*
 * gdntree_accept_commit_build_shared - gdntree_accept_commit_build with the next step's trees
 * built under one batch budget: the same launch (acceptance, commit, per-request builds, here
 * over each request's next_positions[b] positions), then the cut of every next_tree.n_nodes[b]
 * to the request's drafts among the batch's first next_G (as gdntree_build_shared).  For
 * callers that build under a shared budget every step (SpecPilot summary, Technical novelty,
 * batching).  Bitwise the same results as gdntree_accept_commit followed by
 * gdntree_build_shared.
 *
 *   next_positions i32 [next_B] or NULL, next_G >= 0   as for gdntree_build_shared
 *   the rest as for gdntree_accept_commit_build; the limits of gdntree_build_shared apply to
 *   next_B, next_N and next_G.
 */
gdntree_status gdntree_accept_commit_build_shared(
    gdntree_tree tree, int B, int N, int P, const int32_t *target_argmax, int L, int H, int dk,
    int dv, gdntree_dtype in_dtype, const void *k, const void *v, const void *alpha,
    const void *beta, float *state, int32_t *acc_len, int32_t *acc_tok, int32_t *acc_node,
    const float *next_lat_logp, const int32_t *next_lat_tok, const int32_t *next_root_tok,
    const int32_t *next_positions, int next_B, int next_P, int next_K, int next_N, int next_G,
    gdntree_tree next_tree, hipStream_t stream);

/*
 * gdntree_accept_build - gdntree_accept for this step and gdntree_build for the next step's
 * lattices in ONE launch: request b's next tree is built by the workgroup that has just
 * walked request b's acceptance, and no state is touched.  It pairs with
 * gdntree_accept_commit_verify, which commits this step's states inside the next step's
 * verify.  Results are exactly those of gdntree_accept followed by gdntree_build.
 *
 *   tree ... acc_node      as for gdntree_accept (this step)
 *   next_lat_logp ... next_N, next_tree   as for gdntree_build (the next step)
 * next_tree must not share memory with tree; equal parent, token or n_nodes pointers give
 * ERR_ARG.  Every check of the two calls applies; on any error nothing is enqueued.
 */
gdntree_status gdntree_accept_build(gdntree_tree tree, int B, int N, int P,
                                    const int32_t *target_argmax, int32_t *acc_len, int32_t *acc_tok,
                                    int32_t *acc_node, const float *next_lat_logp,
                                    const int32_t *next_lat_tok, const int32_t *next_root_tok,
                                    int next_B, int next_P, int next_K, int next_N,
                                    gdntree_tree next_tree, hipStream_t stream);

/*
 * gdntree_accept_commit_verify - the previous step's acceptance and commit, deferred into
 * this step's verify: ONE launch in which every (layer, request, head) workgroup first walks
 * its request's acceptance of the previous tree (as gdntree_accept), recomputes the accepted
 * node's state from the committed state along the accepted path (as gdntree_commit: fp32,
 * the gated delta rule row by row) and writes it in place, then verifies this step's tree
 * on that state (as gdntree_verify).  The state is read once and written once per step,
 * instead of read by the commit, written, and read again by the next verify (SpecPilot
 * summary, Technical novelty: states recomputed along root paths, not snapshotted).
 * Results are those of gdntree_accept_commit on the previous step followed by
 * gdntree_verify on this one (the state to fp32 rounding of a different summation order).
 *
 *   prev_tree, prev_N, prev_P       the previous step's tree, its node budget and positions
 *   prev_target_argmax i32 [B][prev_N+1]   the target's argmax after each previous slot
 *   prev_k, prev_v     in_dtype [L][B][prev_N+1][H][d]   the previous step's rows
 *   prev_alpha, prev_beta  in_dtype [L][B][prev_N+1][H]
 *   acc_len, acc_tok, acc_node   the previous step's acceptance, as gdntree_accept writes
 *                    it ([B], [B][prev_P+1], [B][prev_P+1]); all three NULL to skip, else
 *                    all three non-NULL (a mix gives ERR_ARG)
 *   tree ... o       as for gdntree_verify (this step); state is read, committed in place,
 *                    and the verify runs on the committed state
 * A request whose previous n_nodes lies outside [1, prev_N+1] keeps its state (and gets no
 * acceptance output); a request whose current tree is malformed gets the NaN / no-output
 * treatment of gdntree_verify, and its state is still committed.  The previous step's
 * arrays are only read; the acceptance outputs must not overlap any input.  Reads
 * prev_tree.parent, prev_tree.token, prev_tree.n_nodes, tree.parent, tree.anc and
 * tree.n_nodes.  Limits: those of gdntree_verify, and prev_N <= 64, prev_P <= 16.
 */
gdntree_status gdntree_accept_commit_verify(
    gdntree_tree prev_tree, int prev_N, int prev_P, const int32_t *prev_target_argmax,
    const void *prev_k, const void *prev_v, const void *prev_alpha, const void *prev_beta,
    int32_t *acc_len, int32_t *acc_tok, int32_t *acc_node, gdntree_tree tree, int B, int N, int L,
    int H, int dk, int dv, gdntree_dtype in_dtype, const void *q, const void *k, const void *v,
    const void *alpha, const void *beta, float *state, gdntree_dtype out_dtype, void *o,
    hipStream_t stream);

/* Human-readable name of a status code ("unknown status" for other values). */
const char *gdntree_status_str(gdntree_status status);

#ifdef __cplusplus
}
#endif

#endif /* GDNTREE_H */
