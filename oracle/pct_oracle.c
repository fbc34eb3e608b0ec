/*
 * pct_oracle.c -- CPU oracle (test infrastructure only; see pct_oracle.h).
 *
 * Plain single-threaded C99, built with -O2 -ffp-contract=off and no
 * fast-math, IEEE round-to-nearest-even.  fp32 steps are written as single
 * fp32 operations so that every rounding point is visible; sums that the
 * method defines exactly (Markov dot products, log-sum-exp, the throughput
 * scan) are taken in double.
 */
#include "pct_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#define REF_OK 0
#define REF_EINVAL 1
#define REF_ENOMEM 2

/* ------------------------------------------------------------------ */
/* inputs                                                              */

static double bf16_bits_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static double factor_at(const void* p, int32_t dtype, int64_t i) {
  if (dtype == REF_BF16) return bf16_bits_to_double(((const uint16_t*)p)[i]);
  return (double)((const float*)p)[i];
}

/* [PCT] "straight draft": the Markov head adds a term that depends on the previous
 * token only.  Stand-in: Markov(t)[v] = sum_j U[t][j] W[v][j]. */
int ref_markov_row(const void* U, const void* W, int32_t uw_dtype, int32_t V,
                   int32_t r, int32_t tok, float* out) {
  if (!U || !W || !out || V < 1 || r < 1 || tok < 0 || tok >= V)
    return REF_EINVAL;
  for (int32_t v = 0; v < V; ++v) {
    double acc = 0.0;
    for (int32_t j = 0; j < r; ++j)
      acc += factor_at(U, uw_dtype, (int64_t)tok * r + j) *
             factor_at(W, uw_dtype, (int64_t)v * r + j);
    out[v] = (float)acc;
  }
  return REF_OK;
}

/* ------------------------------------------------------------------ */
/* per-parent log-softmax and local top-k                              */

typedef struct {
  float z;
  int32_t v;
} zv_t;

/* (z desc, token asc) */
static int cmp_zv(const void* a, const void* b) {
  const zv_t* x = (const zv_t*)a;
  const zv_t* y = (const zv_t*)b;
  if (x->z > y->z) return -1;
  if (x->z < y->z) return 1;
  return (x->v > y->v) - (x->v < y->v);
}

/* [PCT] "straight draft": pi(.|p) is the softmax of z_d(p) = L_d + Markov(p);
 * each parent keeps its local top-k children. */
int ref_row_stats(const float* Lrow, const float* Mrow, int32_t V, int32_t k,
                  float* lse, int32_t* topk_tok, float* topk_z,
                  double* min_gap) {
  if (!Lrow || V < 1 || k < 1 || k > V) return REF_EINVAL;
  zv_t* zs = (zv_t*)malloc(sizeof(zv_t) * (size_t)V);
  if (!zs) return REF_ENOMEM;
  float m = -INFINITY;
  for (int32_t v = 0; v < V; ++v) {
    float z = Mrow ? Lrow[v] + Mrow[v] : Lrow[v]; /* one fp32 add */
    zs[v].z = z;
    zs[v].v = v;
    if (z > m) m = z;
  }
  double s = 0.0;
  for (int32_t v = 0; v < V; ++v) s += exp((double)zs[v].z - (double)m);
  if (lse) *lse = (float)((double)m + log(s));
  qsort(zs, (size_t)V, sizeof(zv_t), cmp_zv);
  for (int32_t i = 0; i < k; ++i) {
    if (topk_tok) topk_tok[i] = zs[i].v;
    if (topk_z) topk_z[i] = zs[i].z;
  }
  if (min_gap) {
    double g = INFINITY;
    int32_t last = k < V ? k : V - 1;
    for (int32_t i = 0; i < last; ++i) {
      double d = (double)zs[i].z - (double)zs[i + 1].z;
      if (d < g) g = d;
    }
    *min_gap = g;
  }
  free(zs);
  return REF_OK;
}

/* ------------------------------------------------------------------ */
/* parent-conditioned tree                                             */

typedef struct {
  float s;      /* path score */
  int32_t ppid; /* parent's pool id (-1 = root) */
  int32_t tok;
  int32_t id;   /* own pool id */
  int32_t depth;
} cand_t;

/* key K = (s desc, parent pool id asc, token asc) */
static int cmp_cand(const void* a, const void* b) {
  const cand_t* x = (const cand_t*)a;
  const cand_t* y = (const cand_t*)b;
  if (x->s > y->s) return -1;
  if (x->s < y->s) return 1;
  if (x->ppid != y->ppid) return x->ppid < y->ppid ? -1 : 1;
  return (x->tok > y->tok) - (x->tok < y->tok);
}

static int32_t frontier_after(int32_t prev, int32_t k, int32_t beam_w) {
  int64_t c = (int64_t)prev * k;
  return c < beam_w ? (int32_t)c : beam_w;
}

int64_t ref_pool_size(const ref_tree_shape* sh) {
  if (!sh) return -1;
  int64_t pool = 0;
  int32_t f = 1;
  for (int32_t d = 1; d <= sh->B; ++d) {
    pool += (int64_t)f * sh->k;
    f = frontier_after(f, sh->k, sh->beam_w);
  }
  return pool;
}

static void gap_update(double* g, float a, float b) {
  double d = (double)a - (double)b;
  if (d < *g) *g = d;
}

/* [PCT] "straight draft", in the article's order: for every frontier parent
 * p compute z_d(p) = L_d + Markov(p) (one call for the whole frontier), take
 * the per-parent log-softmax and local top-k, score every child by its path
 * log-probability s(c) = s(p) + log pi(c|p), prune each stage to the beam,
 * and finally keep the global top-N of all generated children as the tree
 * that fits the verify budget. */
int ref_build_tree(const ref_tree_shape* sh, const float* L, const void* U,
                   const void* W, const int32_t* anchor, int32_t* tok,
                   int32_t* parent, int32_t* depth, float* score,
                   int32_t* n_nodes, double* min_gap, int32_t* pool_tok,
                   int32_t* pool_ppid, float* pool_score, int32_t* beam_pid,
                   double* depth_gap) {
  if (!sh || !L || !anchor || !tok || !parent || !depth || !score || !n_nodes)
    return REF_EINVAL;
  const int32_t batch = sh->batch, B = sh->B, V = sh->V, r = sh->r,
                k = sh->k, Wb = sh->beam_w, N = sh->N;
  if (batch < 1 || B < 1 || V < 1 || k < 1 || k > V || Wb < 1 || N < 1)
    return REF_EINVAL;
  if ((U == NULL) != (W == NULL)) return REF_EINVAL;
  if (U && r < 1) return REF_EINVAL;
  const int64_t pool_n = ref_pool_size(sh);

  cand_t* pool = (cand_t*)malloc(sizeof(cand_t) * (size_t)pool_n);
  cand_t* sorted = (cand_t*)malloc(sizeof(cand_t) * (size_t)pool_n);
  cand_t* front = (cand_t*)malloc(sizeof(cand_t) * (size_t)(Wb + 1));
  float* mrow = U ? (float*)malloc(sizeof(float) * (size_t)V) : NULL;
  int32_t* ktok = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
  float* kz = (float*)malloc(sizeof(float) * (size_t)k);
  int32_t* inv = (int32_t*)malloc(sizeof(int32_t) * (size_t)pool_n);
  if (!pool || !sorted || !front || (U && !mrow) || !ktok || !kz || !inv) {
    free(pool); free(sorted); free(front); free(mrow); free(ktok); free(kz);
    free(inv);
    return REF_ENOMEM;
  }

  int rc = REF_OK;
  for (int32_t q = 0; q < batch && rc == REF_OK; ++q) {
    double gap = INFINITY;
    /* F_0 = the anchor, the root of the tree */
    int32_t nf = 1;
    front[0].s = 0.0f;
    front[0].ppid = -2;
    front[0].tok = anchor[q];
    front[0].id = -1;
    front[0].depth = 0;
    if (anchor[q] < 0 || anchor[q] >= V) { rc = REF_EINVAL; break; }
    int32_t base = 0;
    for (int32_t d = 1; d <= B; ++d) {
      const float* Lrow = L + ((int64_t)q * B + (d - 1)) * V;
      /* expand every frontier parent */
      for (int32_t j = 0; j < nf; ++j) {
        float lse;
        double g;
        if (U) {
          rc = ref_markov_row(U, W, sh->uw_dtype, V, r, front[j].tok, mrow);
          if (rc) break;
        }
        rc = ref_row_stats(Lrow, mrow, V, k, &lse, ktok, kz, &g);
        if (rc) break;
        if (g < gap) gap = g;
        for (int32_t i = 0; i < k; ++i) {
          float l = kz[i] - lse;       /* log pi(v|p), one fp32 subtraction */
          float s = front[j].s + l;    /* path score, one fp32 addition */
          s = s + 0.0f;                /* -0 -> +0 */
          int32_t id = base + j * k + i;
          pool[id].s = s;
          pool[id].ppid = front[j].id;
          pool[id].tok = ktok[i];
          pool[id].id = id;
          pool[id].depth = d;
        }
      }
      if (rc) break;
      /* per-depth pruning: the beam keeps the top-Wb children by K */
      int32_t nc = nf * k;
      memcpy(sorted, pool + base, sizeof(cand_t) * (size_t)nc);
      qsort(sorted, (size_t)nc, sizeof(cand_t), cmp_cand);
      int32_t nf2 = nc < Wb ? nc : Wb;
      double bgap = INFINITY;
      for (int32_t i = 0; i < nf2 && i + 1 < nc; ++i)
        gap_update(&bgap, sorted[i].s, sorted[i + 1].s);
      if (bgap < gap) gap = bgap;
      if (depth_gap) depth_gap[(int64_t)q * (B + 1) + (d - 1)] = bgap;
      memcpy(front, sorted, sizeof(cand_t) * (size_t)nf2);
      if (beam_pid) {
        int32_t* bp = beam_pid + ((int64_t)q * B + (d - 1)) * Wb;
        for (int32_t i = 0; i < Wb; ++i) bp[i] = i < nf2 ? front[i].id : -2;
      }
      nf = nf2;
      base += nc;
    }
    if (rc) break;
    if (pool_tok || pool_ppid || pool_score) {
      for (int64_t i = 0; i < pool_n; ++i) {
        if (pool_tok) pool_tok[q * pool_n + i] = pool[i].tok;
        if (pool_ppid) pool_ppid[q * pool_n + i] = pool[i].ppid;
        if (pool_score) pool_score[q * pool_n + i] = pool[i].s;
      }
    }
    /* global top-N over every generated child */
    memcpy(sorted, pool, sizeof(cand_t) * (size_t)pool_n);
    qsort(sorted, (size_t)pool_n, sizeof(cand_t), cmp_cand);
    int32_t n = pool_n < N ? (int32_t)pool_n : N;
    double tgap = INFINITY;
    for (int32_t i = 0; i < n && i + 1 < pool_n; ++i)
      gap_update(&tgap, sorted[i].s, sorted[i + 1].s);
    if (tgap < gap) gap = tgap;
    if (depth_gap) depth_gap[(int64_t)q * (B + 1) + B] = tgap;
    for (int64_t i = 0; i < pool_n; ++i) inv[i] = -1;
    for (int32_t i = 0; i < n; ++i) inv[sorted[i].id] = i;
    for (int32_t i = 0; i < N; ++i) {
      int64_t o = (int64_t)q * N + i;
      if (i < n) {
        tok[o] = sorted[i].tok;
        depth[o] = sorted[i].depth;
        score[o] = sorted[i].s;
        if (sorted[i].ppid < 0) {
          parent[o] = -1;
        } else {
          parent[o] = inv[sorted[i].ppid];
          if (parent[o] < 0 || parent[o] >= i) rc = REF_EINVAL; /* not closed */
        }
      } else {
        tok[o] = -1;
        parent[o] = -1;
        depth[o] = 0;
        score[o] = -INFINITY;
      }
    }
    n_nodes[q] = n;
    if (min_gap) min_gap[q] = gap;
  }
  free(pool); free(sorted); free(front); free(mrow); free(ktok); free(kz);
  free(inv);
  return rc;
}

/* [PCT] "straight draft": the chain drafter picks, at every position, the most
 * probable token given the previous one. */
int ref_greedy_chain(int32_t B, int32_t V, int32_t r, const float* L,
                     const void* U, const void* W, int32_t uw_dtype,
                     int32_t anchor, int32_t* chain) {
  if (B < 1 || V < 1 || !L || !chain || anchor < 0 || anchor >= V)
    return REF_EINVAL;
  float* mrow = U ? (float*)malloc(sizeof(float) * (size_t)V) : NULL;
  if (U && !mrow) return REF_ENOMEM;
  int32_t prev = anchor;
  for (int32_t d = 1; d <= B; ++d) {
    const float* Lrow = L + (int64_t)(d - 1) * V;
    if (U) ref_markov_row(U, W, uw_dtype, V, r, prev, mrow);
    int32_t best = 0;
    float bz = U ? Lrow[0] + mrow[0] : Lrow[0];
    for (int32_t v = 1; v < V; ++v) {
      float z = U ? Lrow[v] + mrow[v] : Lrow[v];
      if (z > bz) { bz = z; best = v; }
    }
    chain[d - 1] = best;
    prev = best;
  }
  free(mrow);
  return REF_OK;
}

/* ------------------------------------------------------------------ */
/* greedy best-first tree                                              */

typedef struct {
  float s;
  int32_t pout; /* parent's output index, -1 = root */
  int32_t rank; /* position in the parent's child list, (z desc, tok asc) */
  int32_t tok;
  int32_t depth;
} hnode_t;

/* K' = (s desc, parent output index asc, child rank asc); the child rank
 * orders siblings by (z desc, token asc), so equal logits fall back to the
 * token.  Returns 1 if a goes first. */
static int hfirst(const hnode_t* a, const hnode_t* b) {
  if (a->s != b->s) return a->s > b->s;
  if (a->pout != b->pout) return a->pout < b->pout;
  return a->rank < b->rank;
}

typedef struct {
  hnode_t* a;
  int64_t n, cap;
} heap_t;

static int heap_push(heap_t* h, hnode_t x) {
  if (h->n == h->cap) {
    int64_t nc = h->cap ? h->cap * 2 : 1024;
    hnode_t* na = (hnode_t*)realloc(h->a, sizeof(hnode_t) * (size_t)nc);
    if (!na) return REF_ENOMEM;
    h->a = na;
    h->cap = nc;
  }
  int64_t i = h->n++;
  h->a[i] = x;
  while (i > 0) {
    int64_t p = (i - 1) / 2;
    if (!hfirst(&h->a[i], &h->a[p])) break;
    hnode_t t = h->a[i]; h->a[i] = h->a[p]; h->a[p] = t;
    i = p;
  }
  return REF_OK;
}

static hnode_t heap_pop(heap_t* h) {
  hnode_t top = h->a[0];
  h->a[0] = h->a[--h->n];
  int64_t i = 0;
  for (;;) {
    int64_t l = 2 * i + 1, rr = l + 1, m = i;
    if (l < h->n && hfirst(&h->a[l], &h->a[m])) m = l;
    if (rr < h->n && hfirst(&h->a[rr], &h->a[m])) m = rr;
    if (m == i) break;
    hnode_t t = h->a[i]; h->a[i] = h->a[m]; h->a[m] = t;
    i = m;
  }
  return top;
}

/* Push the children of a node (token ptok at depth pdepth, score ps, output
 * index pout).  Children come from depth pdepth+1's row, conditioned on ptok
 * when the Markov factors are given. */
static int push_children(heap_t* h, int32_t B, int32_t V, int32_t r,
                         const float* L, const void* U, const void* W,
                         int32_t dt, int32_t kk, float* mrow,
                         int32_t* ktok, float* kz, int32_t ptok, float ps,
                         int32_t pout, int32_t pdepth, const float* mlse,
                         int32_t* const* mtok, float* const* mz,
                         double* gap) {
  int32_t d = pdepth + 1;
  if (d > B) return REF_OK;
  const float* Lrow = L + (int64_t)(d - 1) * V;
  float lse;
  const int32_t* ct;
  const float* cz;
  if (U) {
    double g;
    int rc = ref_markov_row(U, W, dt, V, r, ptok, mrow);
    if (rc) return rc;
    rc = ref_row_stats(Lrow, mrow, V, kk, &lse, ktok, kz, &g);
    if (rc) return rc;
    if (g < *gap) *gap = g;
    ct = ktok;
    cz = kz;
  } else {
    lse = mlse[d - 1];
    ct = mtok[d - 1];
    cz = mz[d - 1];
  }
  for (int32_t i = 0; i < kk; ++i) {
    hnode_t c;
    float l = cz[i] - lse;
    c.s = ps + l;
    c.s = c.s + 0.0f;
    c.pout = pout;
    c.rank = i;
    c.tok = ct[i];
    c.depth = d;
    int rc = heap_push(h, c);
    if (rc) return rc;
  }
  return REF_OK;
}

/* [CAD] "Method": for a fixed node count the best tree is the greedy
 * best-first one that always adds the prefix of highest probability.  The
 * probability of a prefix is the product of the per-depth probabilities
 * along it (marginals of a block-diffusion drafter when U/W are NULL; the
 * parent-conditioned pi of [PCT] otherwise). */
int ref_bestfirst(int32_t B, int32_t V, int32_t r, const float* L,
                  const void* U, const void* W, int32_t uw_dtype,
                  int32_t anchor, int32_t n_max, int32_t* tok,
                  int32_t* parent, int32_t* depth, float* score,
                  int32_t* n_out, double* min_gap) {
  if (B < 1 || V < 1 || n_max < 1 || !L || !tok || !parent || !depth ||
      !score || !n_out)
    return REF_EINVAL;
  if ((U == NULL) != (W == NULL)) return REF_EINVAL;
  if (U && (anchor < 0 || anchor >= V || r < 1)) return REF_EINVAL;
  const int32_t kk = n_max < V ? n_max : V;
  int rc = REF_OK;
  double gap = INFINITY;
  float* mrow = U ? (float*)malloc(sizeof(float) * (size_t)V) : NULL;
  int32_t* ktok = (int32_t*)malloc(sizeof(int32_t) * (size_t)kk);
  float* kz = (float*)malloc(sizeof(float) * (size_t)kk);
  float* mlse = (float*)malloc(sizeof(float) * (size_t)B);
  int32_t** mtok = (int32_t**)calloc((size_t)B, sizeof(int32_t*));
  float** mz = (float**)calloc((size_t)B, sizeof(float*));
  heap_t h = {NULL, 0, 0};
  if ((U && !mrow) || !ktok || !kz || !mlse || !mtok || !mz) rc = REF_ENOMEM;
  if (!rc && !U) {
    /* marginal rows do not depend on the parent: one set per depth */
    for (int32_t d = 0; d < B && !rc; ++d) {
      double g;
      mtok[d] = (int32_t*)malloc(sizeof(int32_t) * (size_t)kk);
      mz[d] = (float*)malloc(sizeof(float) * (size_t)kk);
      if (!mtok[d] || !mz[d]) { rc = REF_ENOMEM; break; }
      rc = ref_row_stats(L + (int64_t)d * V, NULL, V, kk, &mlse[d], mtok[d],
                         mz[d], &g);
      if (g < gap) gap = g;
    }
  }
  if (!rc)
    rc = push_children(&h, B, V, r, L, U, W, uw_dtype, kk, mrow, ktok, kz,
                       anchor, 0.0f, -1, 0, mlse, mtok, mz, &gap);
  int32_t n = 0;
  float prev_s = 0.0f;
  while (!rc && n < n_max && h.n > 0) {
    hnode_t x = heap_pop(&h);
    if (n > 0) gap_update(&gap, prev_s, x.s);
    prev_s = x.s;
    tok[n] = x.tok;
    parent[n] = x.pout;
    depth[n] = x.depth;
    score[n] = x.s;
    rc = push_children(&h, B, V, r, L, U, W, uw_dtype, kk, mrow, ktok, kz,
                       x.tok, x.s, n, x.depth, mlse, mtok, mz, &gap);
    ++n;
  }
  if (!rc && n == n_max && h.n > 0) {
    /* gap between the last kept node and the best one left out */
    hnode_t x = heap_pop(&h);
    gap_update(&gap, prev_s, x.s);
  }
  for (int32_t i = n; i < n_max; ++i) {
    tok[i] = -1;
    parent[i] = -1;
    depth[i] = 0;
    score[i] = -INFINITY;
  }
  *n_out = n;
  if (min_gap) *min_gap = gap;
  free(h.a);
  free(mrow); free(ktok); free(kz); free(mlse);
  if (mtok) for (int32_t d = 0; d < B; ++d) free(mtok[d]);
  if (mz) for (int32_t d = 0; d < B; ++d) free(mz[d]);
  free(mtok); free(mz);
  return rc;
}

/* ------------------------------------------------------------------ */
/* adaptive budget                                                      */

static double round_cost(const ref_cost_model* c, double n, double ell) {
  return c->C_d + c->c0 + c->c1 * n + c->c2 * n * n + c->c_ell * ell * n;
}

/* [CAD] "Method": maximise (1 + Phi(T_n)) / (C_d + C_v(n; l)) over the
 * trees T_n of the first n nodes of a best-first order; nodes are added in
 * order and the build stops as soon as the marginal gain of the next node
 * is not positive.  The gain of node n+1 has the sign of f(n+1) - f(n),
 * i.e. of P_{n+1} D(n) - (1 + Phi_n)(D(n+1) - D(n)). */
int ref_stop(int32_t n_avail, const float* score, int32_t ctx_len,
             const ref_cost_model* cost, int32_t* n_star, double* phi,
             double* throughput, double* gain_margin) {
  if (!n_star || !phi || !throughput || n_avail < 0 ||
      (n_avail > 0 && !score))
    return REF_EINVAL;
  int32_t ns = n_avail;
  double margin = INFINITY;
  if (cost) {
    const double ell = (double)ctx_len;
    double run = 0.0;
    for (int32_t n = 0; n < n_avail; ++n) {
      double P1 = exp((double)score[n]); /* P_{n+1} (score index n) */
      double Dn = round_cost(cost, (double)n, ell);
      double Dn1 = round_cost(cost, (double)(n + 1), ell);
      double a = P1 * Dn, b = (1.0 + run) * (Dn1 - Dn);
      double g = a - b;
      double den = a > b ? a : b;
      double rel = den > 0 ? fabs(g) / den : INFINITY;
      if (g <= 0.0) {
        ns = n;
        if (rel < margin) margin = rel;
        break;
      }
      /* remember the margin of the last positive gain (n* - 1) */
      margin = rel;
      run += P1;
    }
  }
  double Phi = 0.0;
  for (int32_t i = 0; i < ns; ++i) Phi += exp((double)score[i]);
  *n_star = ns;
  *phi = Phi;
  /* without a cost model the throughput is reported as 1 + Phi */
  *throughput =
      (1.0 + Phi) / (cost ? round_cost(cost, (double)ns, (double)ctx_len)
                          : 1.0);
  if (gain_margin) *gain_margin = margin;
  return REF_OK;
}

/* [CAD] "Method": the throughput of the tree of the first n nodes,
 * f(n) = (1 + Phi_n) / D(n), for every n = 0..n_avail (Phi_n summed in
 * order, in double; D = 1 without a cost model). */
int ref_throughput_curve(int32_t n_avail, const float* score, int32_t ctx_len,
                         const ref_cost_model* cost, double* f) {
  if (!f || n_avail < 0 || (n_avail > 0 && !score)) return REF_EINVAL;
  double Phi = 0.0;
  for (int32_t n = 0; n <= n_avail; ++n) {
    const double D =
        cost ? round_cost(cost, (double)n, (double)ctx_len) : 1.0;
    f[n] = (1.0 + Phi) / D;
    if (n < n_avail) Phi += exp((double)score[n]);
  }
  return REF_OK;
}

/* [CAD] "Method" on the best-first tree: over a block-diffusion drafter's
 * marginals (U, W NULL) or over the parent-conditioned rows of [PCT]
 * "straight draft" (U, W given, the first parent being the anchor). */
int ref_adaptive(int32_t B, int32_t V, int32_t r, int32_t n_max,
                 const float* L, const void* U, const void* W,
                 int32_t uw_dtype, int32_t anchor, int32_t ctx_len,
                 const ref_cost_model* cost, int32_t* tok, int32_t* parent,
                 int32_t* depth, float* score, int32_t* n_star, double* phi,
                 double* throughput, double* min_gap, double* gain_margin) {
  if (!n_star || !phi || !throughput || n_max < 1) return REF_EINVAL;
  int32_t n_avail = 0;
  double gap = INFINITY, order_gap;
  int rc = ref_bestfirst(B, V, r, L, U, W, uw_dtype, anchor, n_max, tok,
                         parent, depth, score, &n_avail, &order_gap);
  if (rc) return rc;
  rc = ref_stop(n_avail, score, ctx_len, cost, n_star, phi, throughput,
                gain_margin);
  if (rc) return rc;
  const int32_t ns = *n_star;
  /* gaps that decide the kept prefix: adjacent scores up to node n*+1 */
  for (int32_t i = 0; i + 1 < n_avail && i <= ns; ++i)
    gap_update(&gap, score[i], score[i + 1]);
  for (int32_t i = ns; i < n_max; ++i) {
    tok[i] = -1;
    parent[i] = -1;
    depth[i] = 0;
    score[i] = -INFINITY;
  }
  if (min_gap) *min_gap = gap;
  return REF_OK;
}

/* ------------------------------------------------------------------ */
/* verification                                                         */

/* [PCT] "straight draft": the whole tree is checked in one target forward;
 * each node may attend to itself and its ancestors only. */
void ref_mask(int32_t N, int32_t n_nodes, const int32_t* parent,
              uint64_t* mask) {
  const int32_t words = (N + 63) / 64;
  memset(mask, 0, sizeof(uint64_t) * (size_t)N * (size_t)words);
  for (int32_t i = 0; i < n_nodes && i < N; ++i) {
    uint64_t* row = mask + (int64_t)i * words;
    int32_t steps = 0;
    for (int32_t a = i; a >= 0 && steps <= N; a = parent[a], ++steps)
      row[a / 64] |= (uint64_t)1 << (a % 64);
  }
}

/* [DSP] "one inference, from guess to confirmation": walk from the root, accept the child whose
 * token equals the target's choice, stop at the first mismatch; the target's
 * own token there is the bonus.  tau counts accepted tokens plus the bonus. */
int ref_accept(int32_t N, int32_t n_nodes, int32_t B, const int32_t* tok,
               const int32_t* parent, const int32_t* target, int32_t* tau,
               int32_t* accept_node, int32_t* accept_tok) {
  if (!tok || !parent || !target || !tau || !accept_node || !accept_tok ||
      n_nodes > N || B < 1)
    return REF_EINVAL;
  for (int32_t i = 0; i < B; ++i) accept_node[i] = -1;
  for (int32_t i = 0; i <= B; ++i) accept_tok[i] = -1;
  int32_t cur = -1, a = 0;
  for (;;) {
    int32_t want = target[cur + 1];
    int32_t next = -1;
    for (int32_t i = 0; i < n_nodes; ++i) {
      if (parent[i] == cur && tok[i] == want) { next = i; break; }
    }
    if (next < 0 || a >= B) break;
    accept_node[a] = next;
    accept_tok[a] = tok[next];
    ++a;
    cur = next;
  }
  accept_tok[a] = target[cur + 1];
  *tau = a + 1;
  return REF_OK;
}

/* ------------------------------------------------------------------ */
/* sampling verification                                               */

/* SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
 * generators", 2014): the finaliser applied to a counter. */
static uint64_t sm64(uint64_t x) {
  x += 0x9E3779B97F4A7C15ull;
  x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
  x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
  return x ^ (x >> 31);
}

double ref_uniform(uint64_t seed, uint64_t stream, uint64_t idx) {
  const uint64_t h = sm64(sm64(sm64(seed) ^ stream) ^ idx);
  return ((double)(h >> 11) + 0.5) * (1.0 / 9007199254740992.0);
}

/* The target's token after each node, sampled at temperature T instead of
 * taken as the argmax (sampling rather than greedy decoding; the pages
 * evaluate greedy decoding only).  Row i of logits [n_rows][V] is the
 * target's distribution after node i-1 (row 0: after the root).  The sample
 * is the Gumbel-max choice argmax_v (z_v / T + G_v), G_v = -log(-log(u_v)),
 * u_v = the counter-based uniform of (seed, stream0 + i, v); ties go to the
 * lowest token.  All in double; 1/T is computed once.  key_gap (optional)
 * receives, per row, the gap between its best and second-best keys. */
int ref_sample_targets(int32_t n_rows, int32_t V, const float* logits,
                       double temperature, uint64_t seed, uint64_t stream0,
                       int32_t* out, double* key_gap) {
  if (n_rows < 0 || V < 1 || !logits || !out || !(temperature > 0.0) ||
      !isfinite(temperature))
    return REF_EINVAL;
  const double inv = 1.0 / temperature;
  for (int32_t i = 0; i < n_rows; ++i) {
    const float* z = logits + (int64_t)i * V;
    double best = -INFINITY, second = -INFINITY;
    int32_t bv = 0;
    for (int32_t v = 0; v < V; ++v) {
      const double u = ref_uniform(seed, stream0 + (uint64_t)i, (uint64_t)v);
      const double g = -log(-log(u));
      const double key = (double)z[v] * inv + g;
      if (key > best) {
        second = best;
        best = key;
        bv = v;
      } else if (key > second) {
        second = key;
      }
    }
    out[i] = bv;
    if (key_gap) key_gap[i] = best - second;
  }
  return REF_OK;
}

