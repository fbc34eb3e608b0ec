/*
 * pct_oracle.h -- CPU oracle for parent-conditioned draft-tree construction.
 *
 * TEST INFRASTRUCTURE ONLY.  This is a plain, slow, single-threaded C
 * implementation of what the GPU library computes.  It exists to check the
 * GPU path; nothing in the product path may link, load or call it.  Only the
 * test-suite, the smoke check and the CPU-baseline leg of the benchmark use it.
 * It shares no code, header, table or helper with the GPU library.
 *
 * Sources (cited by page title and section):
 *  [PCT]  "PCTree" practitioner article on qiita (okssusucha), section
 *         "a straight draft is wasted once its first token misses" (cited
 *         as "straight draft"): the Markov head z_d = L_d + Markov(y_{d-1})
 *         and the chain -> tree step (z_d(p) = L_d + Markov(p) for all
 *         frontier parents,
 *         per-parent log-softmax and local top-k, path score
 *         s(c) = sum log pi(v|u), top-k pruning per stage, global top-N under
 *         the verify budget, one verification forward over the tree).
 *  [DSP]  DSpark explainer (xiaohu-jiedu), section "one inference, from guess to
 *         confirmation":
 *         compare in order, keep consecutive matches, stop at the first
 *         mismatch, the target supplies its own token there (bonus); worked
 *         example of 4 accepted + 1 corrected token.
 *  [CAD]  CaDDTree summary (gist.science 2606.01813), section "Method":
 *         round cost C_d + C_v(|T|; l), objective (1 + Phi(T)) / cost,
 *         greedy best-first tree (highest prefix probability) optimal for a
 *         fixed node count, unimodality under convex C_v, stop when the
 *         marginal gain turns non-positive.
 *
 * Readings where the pages are silent (also listed in the design notes):
 *  - Markov(p) = U[p] . W, low rank, the same for every depth; W is stored
 *    vocab-major: W[v*r + j].
 *  - B drafted positions; depth d uses logit row d-1 of the block; the depth-1
 *    parent is the anchor token.
 *  - pi is the softmax over the whole vocabulary of z; lse in double, rounded
 *    once to fp32; child log-prob l = fp32(z - lse); s = fp32(s(p) + l).
 *  - key K = (s desc, parent pool id asc, token asc); pool ids are depth-major
 *    (base_d + j*k + i); the root's id is -1.
 *  - the candidate pool for the global top-N is every generated child, the
 *    per-depth beam only decides which children are expanded.
 *  - N counts draft nodes only; the root (anchor) is not a node.
 */
#ifndef PCT_ORACLE_H
#define PCT_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { REF_F32 = 0, REF_BF16 = 1 };

typedef struct {
  int32_t batch, B, V, r, k, beam_w, N;
  int32_t uw_dtype; /* REF_F32 or REF_BF16 (U and W stored as raw bf16 bits) */
} ref_tree_shape;

typedef struct {
  double C_d, c0, c1, c2, c_ell; /* C_v(n; l) = c0 + c1 n + c2 n^2 + c_ell l n */
} ref_cost_model;

/* Markov row of token tok: out[v] = fp32(sum_j U[tok][j] * W[v][j]) summed in
 * double (products of bf16 or fp32 inputs are exact in double). */
int ref_markov_row(const void* U, const void* W, int32_t uw_dtype, int32_t V,
                   int32_t r, int32_t tok, float* out);

/* Per-parent statistics of z = fp32(Lrow + Mrow) (Mrow NULL => z = Lrow):
 * lse (fp32 of a double log-sum-exp), the k best tokens by (z desc, token asc)
 * and their z.  min_gap (optional) receives the smallest z gap between
 * adjacent entries of the first min(k+1, V) sorted values. */
int ref_row_stats(const float* Lrow, const float* Mrow, int32_t V, int32_t k,
                  float* lse, int32_t* topk_tok, float* topk_z, double* min_gap);

/* Number of candidates generated per request (the pool). */
int64_t ref_pool_size(const ref_tree_shape* sh);

/* Parent-conditioned tree.  L [batch][B][V]; U, W [V][r] or both NULL (then
 * z = L).  Outputs [batch][N] in K order; parent = output index of the parent
 * (-1 = root); pads beyond n_nodes: tok -1, parent -1, depth 0, score -inf.
 * Optional diagnostics: min_gap [batch]; pool_* [batch][pool] (the generated
 * candidates by pool id); beam_pid [batch][B][beam_w] (the expanded frontier
 * of every depth by pool id, -2 padded); depth_gap [batch][B+1]: entry d-1
 * the smallest score gap between adjacent candidates among the first
 * beam_w+1 of depth d (the beam boundary), entry B the same over the first
 * N+1 of the pool (the global top-N). */
int ref_build_tree(const ref_tree_shape* sh, const float* L, const void* U,
                   const void* W, const int32_t* anchor, int32_t* tok,
                   int32_t* parent, int32_t* depth, float* score,
                   int32_t* n_nodes, double* min_gap, int32_t* pool_tok,
                   int32_t* pool_ppid, float* pool_score, int32_t* beam_pid,
                   double* depth_gap);

/* Greedy chain of the Markov-head drafter: y_0 = anchor,
 * y_d = argmax_v z_d(y_{d-1}) (lowest token on ties). */
int ref_greedy_chain(int32_t B, int32_t V, int32_t r, const float* L,
                     const void* U, const void* W, int32_t uw_dtype,
                     int32_t anchor, int32_t* chain);

/* Greedy best-first tree of one request: repeatedly take the prefix with the
 * highest probability, key K' = (s desc, parent output index asc, child rank
 * asc), where the child rank orders siblings by (z desc, token asc).
 * U/W NULL => marginal rows (block-diffusion drafter); otherwise children are
 * conditioned on the parent token.  Children are restricted to the
 * min(n_max, V) best tokens of their row (exact: a prefix among the n best has
 * rank <= n among its siblings).  Writes up to n_max nodes, *n_out of them. */
int ref_bestfirst(int32_t B, int32_t V, int32_t r, const float* L,
                  const void* U, const void* W, int32_t uw_dtype,
                  int32_t anchor, int32_t n_max, int32_t* tok,
                  int32_t* parent, int32_t* depth, float* score,
                  int32_t* n_out, double* min_gap);

/* Throughput stop over an ordered list of prefix scores (a best-first
 * order): P_i = exp(s_i), Phi_n = sum_{i<=n} P_i, D(n) = C_d + C_v(n; l),
 * g(n) = P_{n+1} D(n) - (1 + Phi_n)(D(n+1) - D(n)); n* is the first n with
 * g(n) <= 0 (n_avail if none; cost NULL => n_avail).  Outputs n*,
 * Phi(n*), the throughput (1 + Phi)/D(n*) (1 + Phi without a cost model)
 * and, optionally, gain_margin = min over n in {n*-1, n*} of
 * |g(n)| / max(P_{n+1} D(n), (1+Phi_n) dD(n)). */
int ref_stop(int32_t n_avail, const float* score, int32_t ctx_len,
             const ref_cost_model* cost, int32_t* n_star, double* phi,
             double* throughput, double* gain_margin);

/* f(n) = (1 + Phi_n) / D(n) for n = 0..n_avail (f has n_avail + 1
 * entries; D = 1 without a cost model). */
int ref_throughput_curve(int32_t n_avail, const float* score, int32_t ctx_len,
                         const ref_cost_model* cost, double* f);

/* Adaptive best-first tree: ref_bestfirst (marginal rows when U/W are NULL,
 * parent-conditioned rows from the anchor otherwise) followed by ref_stop.
 * Writes the first n* nodes (pads as in ref_build_tree), n*, Phi(n*), the
 * throughput, and optionally the smallest adjacent score gap up to node
 * n*+1 (min_gap) and the gain margin. */
int ref_adaptive(int32_t B, int32_t V, int32_t r, int32_t n_max,
                 const float* L, const void* U, const void* W,
                 int32_t uw_dtype, int32_t anchor, int32_t ctx_len,
                 const ref_cost_model* cost, int32_t* tok, int32_t* parent,
                 int32_t* depth, float* score, int32_t* n_star, double* phi,
                 double* throughput, double* min_gap, double* gain_margin);

/* Packed ancestry mask of one tree: row i holds bit i and every bit of its
 * ancestors; words per row = ceil(N/64), bit j%64 of word j/64; rows >= n
 * are zero. */
void ref_mask(int32_t N, int32_t n_nodes, const int32_t* parent,
              uint64_t* mask);

/* Greedy acceptance walk of one tree.  target [N+1]: target[0] is the
 * target's token after the root, target[1+i] after node i.  Outputs tau =
 * accepted + 1, accept_node [B] (-1 padded) and accept_tok [B+1]
 * (accepted tokens, then the target's own token, -1 padded). */
int ref_accept(int32_t N, int32_t n_nodes, int32_t B, const int32_t* tok,
               const int32_t* parent, const int32_t* target, int32_t* tau,
               int32_t* accept_node, int32_t* accept_tok);

/* Counter-based uniform in (0, 1): SplitMix64 of (seed, stream, idx),
 * ((h >> 11) + 0.5) * 2^-53 with h = sm(sm(sm(seed) ^ stream) ^ idx). */
double ref_uniform(uint64_t seed, uint64_t stream, uint64_t idx);

/* Sampled target tokens: row i of logits [n_rows][V] gives
 * out[i] = argmax_v (z_v / T - log(-log(u(seed, stream0 + i, v)))), ties to
 * the lowest token (Gumbel-max sampling from softmax(z / T)); key_gap
 * (optional) [n_rows]: best minus second-best key. */
int ref_sample_targets(int32_t n_rows, int32_t V, const float* logits,
                       double temperature, uint64_t seed, uint64_t stream0,
                       int32_t* out, double* key_gap);

#ifdef __cplusplus
}
#endif
#endif
