/*
 * pctree.h -- libpctree: draft-tree construction and checking for
 * speculative decoding, on AMD Instinct MI355X (gfx950).
 *
 * Pages the operations come from (cited by title and section):
 *  [PCT] qiita article on PCTree (Parent-Conditioned Drafting Tree),
 *        section "a straight draft is wasted once its first token misses"
 *        (cited below as "straight draft"): DSpark's Markov head
 *        z_d = L_d + Markov(y_{d-1}) and the chain -> tree step.
 *  [DSP] DSpark / DeepSeek-V4 explainer (xiaohu-jiedu), section "one
 *        inference, from guess to confirmation".
 *  [CAD] "Cost-Aware Diffusion Draft Trees for Speculative Decoding"
 *        (CaDDTree) summary on gist.science, section "Method".
 *
 * Conventions shared by every call
 *  - Pointers are DEVICE pointers unless marked (host).  Every call is
 *    asynchronous on `stream` (a hipStream_t passed as void*; NULL = the
 *    default stream) and never synchronises the host.
 *  - The caller owns every buffer, including the workspace, and keeps them
 *    alive until the stream has finished the work.  The library allocates
 *    nothing and keeps no pointer after a call returns.
 *  - Arrays are row-major and contiguous.  Token ids are int32 in [0, V),
 *    V < 2^18.  A parent index of -1 means the root (the anchor token); the
 *    root is not one of the N nodes.
 *  - Masks are uint64 words: bit j%64 of word j/64 of row i is set when node
 *    j is node i or one of its ancestors.
 *  - Every argument is checked on the host before anything is enqueued; a
 *    failed check returns a status and enqueues nothing.  A failed launch
 *    returns PCT_ERR_HIP.  pct_last_error() gives the reason (per thread).
 *    No exception crosses this interface and the library never aborts.
 *  - Logits must be finite.
 *  - Calls are reentrant; calls on different streams need different
 *    workspaces.
 */
#ifndef PCTREE_H
#define PCTREE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PCT_OK = 0,
  PCT_ERR_INVALID_ARG = 1,
  PCT_ERR_UNSUPPORTED = 2,
  PCT_ERR_WORKSPACE = 3,
  PCT_ERR_HIP = 4
} pct_status;

typedef enum { PCT_F32 = 0, PCT_BF16 = 1 } pct_dtype;

/* Shape of a parent-conditioned build.
 *  batch   independent requests
 *  B       drafted positions per block (tree depth <= B)
 *  V       vocabulary size
 *  r       rank of the Markov factors (ignored when U and W are NULL)
 *  k       children kept per parent (local top-k)
 *  beam_w  parents expanded per depth and request (per-stage pruning)
 *  N       verify budget: nodes kept per request (global top-N)
 *  uw_dtype  element type of U and W */
typedef struct {
  int32_t batch, B, V, r, k, beam_w, N;
  int32_t uw_dtype;
} pct_tree_shape;

/* Round cost of the adaptive build: C(n; l) = C_d + C_v(n; l) with
 * C_v(n; l) = c0 + c1 n + c2 n^2 + c_ell l n (convex and increasing in n
 * when c1, c2, c_ell >= 0). */
typedef struct {
  double C_d, c0, c1, c2, c_ell;
} pct_cost_model;

/* ------------------------------------------------------------------------
 * pct_markov_logits -- [PCT] "straight draft": for P parents
 * at once, z_p = L[row_p] + Markov(tok_p) with Markov(t)[v] = U[t] . W[v],
 * then the log-softmax normaliser of z_p over the vocabulary and its top-k.
 *
 *  L          [L_rows][L_row_stride] fp32 drafter logits; NULL => z = Markov
 *             (row indices outside [0, L_rows) are clamped; token ids
 *             outside [0, V) are clamped)
 *  U, W       [V][r] Markov factors (W stored vocab-major, i.e. the [r x V]
 *             factor transposed); both NULL => z = L
 *  parent_tok [P] token of each parent; parent_Lrow [P] its L row
 *  lse        [P] out: log sum_v exp(z_p[v])
 *  topk_tok   [P][k] out: tokens by (z desc, token asc)
 *  topk_logp  [P][k] out: z - lse of those tokens
 *  z_out      [P][V] out, optional (NULL in the fast path): the logit rows
 *  workspace  pct_markov_logits_workspace(P, V, k) bytes
 * Errors: PCT_ERR_INVALID_ARG for k < 1, k > V, V >= 2^18, P < 1, null
 * required pointers, or exactly one of U/W NULL; PCT_ERR_UNSUPPORTED for
 * k > 64 or P > 65535; PCT_ERR_WORKSPACE when workspace_bytes is too small.
 * bf16 factors with r in {32, 64, 128, 256} run on MFMA; other ranks and
 * fp32 factors take a plain VALU kernel. */
pct_status pct_markov_logits(const float* L, int64_t L_row_stride,
                             int32_t L_rows, const void* U, const void* W,
                             pct_dtype uw_dtype,
                             int32_t V, int32_t r, const int32_t* parent_tok,
                             const int32_t* parent_Lrow, int32_t P, int32_t k,
                             float* lse, int32_t* topk_tok, float* topk_logp,
                             float* z_out, void* workspace,
                             size_t workspace_bytes, void* stream);
size_t pct_markov_logits_workspace(int32_t P, int32_t V, int32_t k);

/* ------------------------------------------------------------------------
 * pct_build_tree -- [PCT] "straight draft": the parent-conditioned draft tree.
 * Depth d = 1..B expands every frontier parent p with
 * z_d(p) = L_d + Markov(p) (one batched call per depth), keeps each
 * parent's top-k children by log pi(v|p) = z - lse, scores a child by its
 * path log-probability s(c) = s(p) + log pi(c|p), keeps the beam_w best
 * children per request as the next frontier, and finally keeps the N best
 * of all generated children as the tree that fits the verify budget.
 * Order and ties: key (score desc, parent's pool id asc, token asc); the
 * pool id of a child is base_d + j*k + i for the i-th child of the j-th
 * frontier parent; the root's is -1.
 *
 *  L       [batch][B][V] fp32; row d-1 drives depth d
 *  U, W    [V][r] (W vocab-major) or both NULL (then z_d = L_d); both
 *          16-byte aligned
 *  anchor  [batch] root token of each request (the depth-1 parent)
 *  tok, parent, depth  [batch][N] int32 out; score [batch][N] fp32 out.
 *          Nodes come in key order, so parents precede children; parent is
 *          the output index of the parent, -1 for the root.  Entries past
 *          n_nodes hold tok -1, parent -1, depth 0, score -inf.
 *  n_nodes [batch] out: min(N, generated children)
 *  mask    [batch][N][ceil(N/64)] out, optional (NULL = not built)
 *  workspace  pct_build_tree_workspace(shape) bytes
 * Errors: as pct_markov_logits, plus PCT_ERR_INVALID_ARG for U or W not
 * 16-byte aligned, and PCT_ERR_UNSUPPORTED when the pool of generated
 * children per request exceeds 8192 or a per-depth candidate set exceeds
 * 2048. */
pct_status pct_build_tree(const pct_tree_shape* shape /*host*/,
                          const float* L, const void* U, const void* W,
                          const int32_t* anchor, int32_t* tok,
                          int32_t* parent, int32_t* depth, float* score,
                          int32_t* n_nodes, uint64_t* mask, void* workspace,
                          size_t workspace_bytes, void* stream);
size_t pct_build_tree_workspace(const pct_tree_shape* shape /*host*/);

/* ------------------------------------------------------------------------
 * pct_build_tree_adaptive -- [CAD] "Method": the greedy best-first tree
 * over a block-diffusion drafter's per-position marginals with the
 * throughput stop.  The probability of a prefix is the product of its
 * per-depth marginals, log pi_d(v) = L_d[v] - lse_d; nodes are taken in
 * best-first order, key (score desc, parent output index asc, child rank
 * asc), where a child's rank orders its row by (logit desc, token asc), so
 * equal scores fall back to the rank and equal logits to the token;
 * with P_i = exp(score_i), Phi_n = sum_{i<=n} P_i and D(n) = C(n; l), the
 * build stops at the first n whose gain
 * g(n) = P_{n+1} D(n) - (1 + Phi_n)(D(n+1) - D(n)) is not positive, i.e.
 * where (1 + Phi)/D stops increasing.  cost NULL => a fixed budget n_max.
 *
 *  L        [batch][B][V] fp32 marginal logits
 *  ctx_len  [batch] context length l of each request
 *  tok, parent, depth, score  [batch][n_max] out; the first n_star entries
 *           are the tree in best-first order, the rest are pads as above
 *  n_star   [batch] out; phi [batch] out Phi(n*); throughput [batch] out
 *           (1 + Phi)/D(n*) (1 + Phi without a cost model)
 *  mask     [batch][n_max][ceil(n_max/64)] out, optional
 * Every candidate is a child of a taken node among the min(n_max, V) best
 * tokens of its row (a node among the n best prefixes has rank < n among
 * its siblings), so the search is exact.  Each taken node opens at most
 * two candidates (its next sibling and its first child), so the open set
 * stays below 2 n_max + 2 entries.
 * Errors: PCT_ERR_INVALID_ARG for n_max < 1, B < 1, V < 1, V >= 2^18,
 * batch < 1 or null pointers; PCT_ERR_UNSUPPORTED for n_max > 1024 or
 * B > 255; a cost model with negative c1, c2 or c_ell, or with
 * C_d + c0 <= 0, is rejected (the stop rule is only the throughput optimum
 * for a positive, convex, increasing cost). */
pct_status pct_build_tree_adaptive(int32_t batch, int32_t B, int32_t V,
                                   int32_t n_max, const float* L,
                                   const int32_t* ctx_len,
                                   const pct_cost_model* cost /*host*/,
                                   int32_t* tok, int32_t* parent,
                                   int32_t* depth, float* score,
                                   int32_t* n_star, double* phi,
                                   double* throughput, uint64_t* mask,
                                   void* workspace, size_t workspace_bytes,
                                   void* stream);
size_t pct_build_tree_adaptive_workspace(int32_t batch, int32_t B, int32_t V,
                                         int32_t n_max);

/* ------------------------------------------------------------------------
 * pct_build_tree_adaptive_pc -- [CAD] "Method" on the parent-conditioned
 * tree of [PCT] "straight draft": the throughput stop over the key order of
 * a pct_build_tree build.  The build (shape, L, U, W, anchor as for
 * pct_build_tree, with N = n_max, the largest tree considered) yields its
 * nodes in key order, which is a best-first order: every node comes after
 * its parent.  With P_i = exp(score_i), Phi_n = sum_{i<=n} P_i and
 * D(n) = C(n; l), the tree keeps the first n* nodes, n* being the first n
 * whose gain g(n) = P_{n+1} D(n) - (1 + Phi_n)(D(n+1) - D(n)) is not
 * positive.  When k >= n* and beam_w >= n*, the kept nodes are the n* most
 * probable prefixes of the parent-conditioned drafter, i.e. the greedy
 * best-first tree (a top-n prefix has sibling rank < n and depth rank < n,
 * so the beam keeps it); with smaller k or beam_w it is the beam's
 * approximation of it.  cost NULL => n* = the number of nodes built.
 *
 *  tok, parent, depth, score  [batch][N] out: the first n_star entries are
 *           the tree, the rest pads (tok -1, parent -1, depth 0,
 *           score -inf)
 *  ctx_len  [batch] context length l of each request (needed with cost)
 *  n_star   [batch] out; phi [batch] out Phi(n*); throughput [batch] out
 *           (1 + Phi)/D(n*) (1 + Phi without a cost model)
 *  mask     [batch][N][ceil(N/64)] out, optional: the kept tree's mask
 *  workspace  pct_build_tree_adaptive_pc_workspace(shape) bytes
 * Errors: as pct_build_tree; a cost model with negative c1, c2 or c_ell, or
 * with C_d + c0 <= 0, is rejected with PCT_ERR_INVALID_ARG. */
pct_status pct_build_tree_adaptive_pc(
    const pct_tree_shape* shape /*host*/, const float* L, const void* U,
    const void* W, const int32_t* anchor, const int32_t* ctx_len,
    const pct_cost_model* cost /*host*/, int32_t* tok, int32_t* parent,
    int32_t* depth, float* score, int32_t* n_star, double* phi,
    double* throughput, uint64_t* mask, void* workspace,
    size_t workspace_bytes, void* stream);
size_t pct_build_tree_adaptive_pc_workspace(const pct_tree_shape* shape /*host*/);

/* ------------------------------------------------------------------------
 * pct_throughput_curve -- [CAD] "Method": the throughput of every prefix
 * of a best-first-ordered tree, f(n) = (1 + Phi_n) / D(n) for n = 0..N
 * (D = 1 without a cost model), as a fixed-budget (DDTree-style) build of n
 * nodes would get it; the oracle budget of a round is the n that maximises
 * it.  Budgets above a request's n_nodes repeat f(n_nodes).
 *  score    [batch][N] scores in best-first order (e.g. the output of a
 *           build without a cost model), n_nodes [batch]
 *  ctx_len  [batch] (needed with cost)
 *  f        [batch][N+1] out
 * Needs no workspace.
 * Errors: PCT_ERR_INVALID_ARG for batch < 1, N < 1, null required pointers
 * or a cost model that is not convex and increasing. */
pct_status pct_throughput_curve(int32_t batch, int32_t N, const float* score,
                                const int32_t* n_nodes,
                                const int32_t* ctx_len,
                                const pct_cost_model* cost /*host*/,
                                double* f, void* stream);

/* ------------------------------------------------------------------------
 * pct_tree_mask -- [PCT] "straight draft": the whole tree is verified in one
 * target forward, in which a node may see only itself and its ancestors.
 *  parent  [batch][N] (-1 = root), n_nodes [batch]
 *  mask    [batch][N][ceil(N/64)] out; rows >= n_nodes are zero
 * Errors: PCT_ERR_INVALID_ARG for batch < 1, N < 1 or null pointers. */
pct_status pct_tree_mask(int32_t batch, int32_t N, const int32_t* parent,
                         const int32_t* n_nodes, uint64_t* mask,
                         void* stream);

/* ------------------------------------------------------------------------
 * pct_verify_accept -- [DSP] "one inference, from guess to confirmation":
 * compare the draft with the target in order, accept the run of matches,
 * stop at the first mismatch where the target supplies its own token.  On
 * a tree: a node is accepted when its token equals the target's choice
 * after its parent and its parent is accepted (the root always is).
 *
 *  tok, parent, depth [batch][N] tree (parents precede children; siblings
 *          carry distinct tokens), n_nodes [batch]
 *  mask    [batch][N][ceil(N/64)] optional: the tree's packed ancestry mask
 *          (as pct_tree_mask writes it).  When given, a node is accepted
 *          exactly when every node of its mask row matches, which replaces
 *          the walk up the parent links by word operations; NULL = walk
 *  target  [batch][N+1]: target[0] is the target's token after the root,
 *          target[1+i] its token after node i
 *  tau     [batch] out: accepted tokens + 1 (the target's own token)
 *  accept_node [batch][B] out: the accepted nodes root-to-leaf, -1 padded
 *  accept_tok  [batch][B+1] out: their tokens, then the target's token,
 *          -1 padded
 * Needs no workspace.
 * Errors: PCT_ERR_INVALID_ARG for batch < 1, N < 1, B < 1, N > 8192 or
 * null required pointers. */
pct_status pct_verify_accept(int32_t batch, int32_t N, int32_t B,
                             const int32_t* tok, const int32_t* parent,
                             const int32_t* depth, const int32_t* n_nodes,
                             const uint64_t* mask, const int32_t* target,
                             int32_t* tau, int32_t* accept_node,
                             int32_t* accept_tok, void* stream);

/* ------------------------------------------------------------------------
 * pct_verify_sample -- verification with temperature sampling instead of
 * greedy decoding.  The pages evaluate greedy decoding only ([PCT] "how
 * well it works, in numbers") and give no sampling rule; this call takes
 * the plainest one that keeps the target's distribution for a tree of
 * fixed (top-k) children: the target's token after each node is a sample
 * from softmax(target logits / T) rather than its argmax, and the walk of
 * pct_verify_accept runs on those samples ([DSP] "one inference, from guess
 * to confirmation": accept while the target's token is a drafted child,
 * then the target's own token).  Every emitted token is a target sample.
 * Sampling is Gumbel-max: token = argmax_v (z_v / T - log(-log(u_v))), ties
 * to the lowest token, keys in double, u_v = ((h >> 11) + 0.5) * 2^-53 with
 * h = sm(sm(sm(seed) ^ stream) ^ v), sm the SplitMix64 finaliser (Steele,
 * Lea and Flood, 2014) and stream = request * (N+1) + row.
 *
 *  tok, parent, depth, n_nodes, mask  the tree, as for pct_verify_accept
 *  target_logits  [batch][N+1][V] fp32: row 0 the target's logits after
 *          the root, row 1+i after node i (rows past n_nodes are not read)
 *  temperature    T > 0; seed  the generator's seed
 *  sampled [batch][N+1] out: the sampled target tokens (-1 past n_nodes)
 *  tau, accept_node, accept_tok  out, as for pct_verify_accept
 *  workspace  device memory of pct_verify_sample_workspace(batch, N, V)
 *          bytes: when there are few rows each row is cut into slices whose
 *          partial arg-maxes land there; may be NULL when that size is 0
 *          (enough rows to fill the GPU one workgroup per row)
 * Errors: PCT_ERR_INVALID_ARG for batch, B or V < 1, N outside [1, 8192],
 * a temperature that is not positive and finite, or null required
 * pointers; PCT_ERR_UNSUPPORTED for batch > 65535; PCT_ERR_WORKSPACE for a
 * missing or short workspace. */
size_t pct_verify_sample_workspace(int32_t batch, int32_t N, int32_t V);
pct_status pct_verify_sample(int32_t batch, int32_t N, int32_t B, int32_t V,
                             const int32_t* tok, const int32_t* parent,
                             const int32_t* depth, const int32_t* n_nodes,
                             const uint64_t* mask, const float* target_logits,
                             double temperature, uint64_t seed,
                             int32_t* sampled, int32_t* tau,
                             int32_t* accept_node, int32_t* accept_tok,
                             void* workspace, size_t workspace_bytes,
                             void* stream);

/* ------------------------------------------------------------------------
 * pct_build_tree_noalloc -- for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): pct_build_tree with the same arguments minus the workspace,
 * which is instead a fixed 32 MiB device array inside the library, one per
 * GPU, held until the process ends.  Shapes whose
 * pct_build_tree_workspace() exceeds 32 MiB return PCT_ERR_UNSUPPORTED
 * before anything is enqueued (the batch-128, N = 512 round needs about
 * 21 MB).  Allocates nothing.  All calls on one GPU share its array, so
 * calls that overlap in time on one GPU (other streams or threads) race;
 * calls ordered on one stream do not.  Errors otherwise as pct_build_tree. */
pct_status pct_build_tree_noalloc(const pct_tree_shape* shape /*host*/,
                                  const float* L, const void* U,
                                  const void* W, const int32_t* anchor,
                                  int32_t* tok, int32_t* parent,
                                  int32_t* depth, float* score,
                                  int32_t* n_nodes, uint64_t* mask,
                                  void* stream);

/* ------------------------------------------------------------------------
 * Profiling (not from the pages; for measuring kernels against the
 * hardware roofline).  When enabled, every kernel launch of the calls above
 * is bracketed by two HIP events recorded on its stream, tagged with a kind
 * and its work units.  Kinds: 0 fused Markov/log-sum-exp/top-k kernel
 * (units = parents of the launch), 1 per-request expand, 2 global top-N,
 * 3 mask, 4 acceptance walk, 5 seed pre-pass (units = rows), 6 depth-1
 * init, 7 adaptive row statistics (units = rows), 8 adaptive best-first +
 * stop, 9 standalone per-parent results, 10 throughput stop / curve scan,
 * 11 sampled target tokens.
 *  pct_profile_enable  turns recording on or off (the event pool, 8192
 *                      launches, is created on the first enable)
 *  pct_profile_reset   forgets recorded launches
 *  pct_profile_read    total milliseconds and number of recorded launches of
 *                      one kind (units < 0: any units); waits for the events
 * Not thread-safe against concurrent calls that launch kernels. */
pct_status pct_profile_enable(int32_t enable);
pct_status pct_profile_reset(void);
pct_status pct_profile_read(int32_t kind, int64_t units, double* total_ms,
                            int64_t* launches);

const char* pct_status_string(pct_status s);
const char* pct_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* PCTREE_H */
