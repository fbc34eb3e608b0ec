// api.hip -- the C-ABI of libpctree: argument checks, workspace carving and
// the launch sequence of every call.  All work is enqueued on the caller's
// stream; nothing here synchronises or allocates.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>

#include "../../include/pctree.h"
#include "pct_internal.h"

using namespace pct;

namespace {

thread_local char g_err[512] = "";

pct_status fail(pct_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

pct_status hip_fail(hipError_t e, const char* what) {
  return fail(PCT_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

// Bump allocator over the caller's workspace.
struct Carve {
  char* base;
  size_t off = 0;
  template <typename T>
  T* take(size_t n) {
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off = align_up(off + n * sizeof(T));
    return p;
  }
};

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

int frontier_after(int prev, int k, int beam_w) {
  const int64_t c = (int64_t)prev * k;
  return c < beam_w ? (int)c : beam_w;
}

// Frontier sizes, pool layout and per-depth fused-kernel plans of a build.
struct TreePlan {
  int F[66];      // F[d] = frontier size after depth d, F[0] = 1
  int base[66];   // pool id where depth d's children start
  int pool_n;
  int Fmax;       // max frontier size over depths 0..B
  K1Plan k1[65];  // plan of depth d
  int max_slices_P;
  int max_cap_P;
  int max_P;
  int max_tq;  // tile-queue counters of the largest fused launch
};

pct_status plan_tree(const pct_tree_shape* sh, TreePlan& tp) {
  const int B = sh->B;
  tp.F[0] = 1;
  tp.Fmax = 1;
  int64_t pool = 0;
  for (int d = 1; d <= B; ++d) {
    tp.base[d] = (int)pool;
    pool += (int64_t)tp.F[d - 1] * sh->k;
    if ((int64_t)tp.F[d - 1] * sh->k > kMaxCand)
      return fail(PCT_ERR_UNSUPPORTED,
                  "children per request at depth %d (%lld) exceed %d", d,
                  (long long)tp.F[d - 1] * sh->k, kMaxCand);
    tp.F[d] = frontier_after(tp.F[d - 1], sh->k, sh->beam_w);
    if (tp.F[d] > tp.Fmax) tp.Fmax = tp.F[d];
  }
  tp.base[B + 1] = (int)pool;
  if (pool > kMaxPool)
    return fail(PCT_ERR_UNSUPPORTED, "pool of %lld children exceeds %d",
                (long long)pool, kMaxPool);
  tp.pool_n = (int)pool;
  const bool has_uw = sh->r > 0;
  if (!has_uw || sh->uw_dtype != PCT_BF16) {
    if ((int64_t)sh->batch * tp.Fmax > 65535)
      return fail(PCT_ERR_UNSUPPORTED, "too many parents per depth");
  }
  tp.max_slices_P = 0;
  tp.max_cap_P = 0;
  tp.max_P = 0;
  tp.max_tq = 0;
  for (int d = 1; d <= B; ++d) {
    // without Markov factors every parent of a request shares its row
    const int P = has_uw ? sh->batch * tp.F[d - 1] : sh->batch;
    tp.k1[d] = plan_k1(P, sh->V, sh->r, sh->k, sh->uw_dtype, has_uw, true,
                       has_uw ? tp.F[d - 1] : 0);
    const int sp = tp.k1[d].n_slices * P;
    const int cp = tp.k1[d].cap * P;
    if (tp.k1[d].n_tq > tp.max_tq) tp.max_tq = tp.k1[d].n_tq;
    if (sp > tp.max_slices_P) tp.max_slices_P = sp;
    if (cp > tp.max_cap_P) tp.max_cap_P = cp;
    if (P > tp.max_P) tp.max_P = P;
  }
  return PCT_OK;
}

struct TreeWs {
  int32_t* rowtop;
  int32_t *ftok[2], *fpid[2], *flrow[2];
  float *fs[2], *ftheta[2];
  float *part_c, *part_s;
  int32_t* gcnt[2];
  float* gz;
  int32_t* gv;
  uint64_t* pool_key;
  uint4* upack;  // packed U rows of one depth's parents (MFMA plans only)
  uint64_t* ckey;  // one depth's child keys (split expand)
  int32_t* tq;     // fused-kernel tile queue (cleared by init)
};

size_t carve_tree(const pct_tree_shape* sh, const TreePlan& tp, void* ws,
                  TreeWs& w) {
  Carve c{static_cast<char*>(ws)};
  const int64_t FB = (int64_t)sh->batch * tp.Fmax;
  w.rowtop = c.take<int32_t>((size_t)sh->batch * sh->B * kSeedT);
  for (int i = 0; i < 2; ++i) {
    w.ftok[i] = c.take<int32_t>(FB);
    w.fpid[i] = c.take<int32_t>(FB);
    w.flrow[i] = c.take<int32_t>(FB);
    w.fs[i] = c.take<float>(FB);
    w.ftheta[i] = c.take<float>(FB);
    w.gcnt[i] = c.take<int32_t>(tp.max_P > FB ? tp.max_P : FB);
  }
  w.part_c = c.take<float>(tp.max_slices_P);
  w.part_s = c.take<float>(tp.max_slices_P);
  w.gz = c.take<float>(tp.max_cap_P);
  w.gv = c.take<int32_t>(tp.max_cap_P);
  w.pool_key = c.take<uint64_t>((size_t)sh->batch * tp.pool_n);
  // packed U rows: whole 32-parent blocks of r/8 16-byte chunks
  const bool mfma = tp.k1[1].kind == K1_MFMA;
  w.upack = c.take<uint4>(mfma ? (size_t)((tp.max_P + 31) / 32 * 32) *
                                     (sh->r / 8)
                               : 0);
  w.ckey = c.take<uint64_t>((size_t)FB * sh->k);
  w.tq = c.take<int32_t>(tp.max_tq);
  return c.off;
}

pct_status check_shape(const pct_tree_shape* sh) {
  if (!sh) return fail(PCT_ERR_INVALID_ARG, "shape is NULL");
  if (sh->batch < 1 || sh->B < 1 || sh->B > 64 || sh->V < 1 || sh->k < 1 ||
      sh->beam_w < 1 || sh->N < 1)
    return fail(PCT_ERR_INVALID_ARG,
                "need batch, B (<= 64), V, k, beam_w, N >= 1");
  if (sh->V >= (1 << 18))
    return fail(PCT_ERR_INVALID_ARG, "V = %d must be below 2^18", sh->V);
  if (sh->k > sh->V) return fail(PCT_ERR_INVALID_ARG, "k > V");
  if (sh->k > kMaxK)
    return fail(PCT_ERR_UNSUPPORTED, "k = %d exceeds %d", sh->k, kMaxK);
  if (sh->uw_dtype != PCT_F32 && sh->uw_dtype != PCT_BF16)
    return fail(PCT_ERR_INVALID_ARG, "unknown factor dtype");
  return PCT_OK;
}

}  // namespace

namespace pct {
pct_status set_error(pct_status st, const char* msg) {
  snprintf(g_err, sizeof g_err, "%s", msg);
  return st;
}
}  // namespace pct

extern "C" {

const char* pct_status_string(pct_status s) {
  switch (s) {
    case PCT_OK: return "ok";
    case PCT_ERR_INVALID_ARG: return "invalid argument";
    case PCT_ERR_UNSUPPORTED: return "unsupported configuration";
    case PCT_ERR_WORKSPACE: return "workspace too small";
    case PCT_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* pct_last_error(void) { return g_err; }

// ------------------------------------------------------------------------
size_t pct_markov_logits_workspace(int32_t P, int32_t V, int32_t k) {
  if (P < 1 || V < 1 || k < 1) return 0;
  // the largest layout over every kernel the call may plan: the MFMA
  // kernel at each supported rank (its shape depends on r through the LDS
  // it needs) and the simple kernel
  K1Plan plans[5] = {plan_k1(P, V, 32, k, PCT_BF16, true),
                     plan_k1(P, V, 64, k, PCT_BF16, true),
                     plan_k1(P, V, 128, k, PCT_BF16, true),
                     plan_k1(P, V, 256, k, PCT_BF16, true),
                     plan_k1(P, V, 0, k, PCT_F32, false)};
  size_t need = 0;
  for (const K1Plan* pl = plans; pl != plans + 5; ++pl) {
    Carve c{nullptr};
    c.take<float>((size_t)pl->n_slices * P);
    c.take<float>((size_t)pl->n_slices * P);
    c.take<int32_t>(P + pl->n_tq);
    c.take<float>((size_t)pl->cap * P);
    c.take<int32_t>((size_t)pl->cap * P);
    if (c.off > need) need = c.off;
  }
  return need;
}

pct_status pct_markov_logits(const float* L, int64_t L_row_stride,
                             int32_t L_rows, const void* U, const void* W,
                             pct_dtype uw_dtype,
                             int32_t V, int32_t r, const int32_t* parent_tok,
                             const int32_t* parent_Lrow, int32_t P, int32_t k,
                             float* lse, int32_t* topk_tok, float* topk_logp,
                             float* z_out, void* workspace,
                             size_t workspace_bytes, void* stream) {
  if (P < 1 || V < 1 || k < 1 || k > V)
    return fail(PCT_ERR_INVALID_ARG, "need P, V >= 1 and 1 <= k <= V");
  if (V >= (1 << 18)) return fail(PCT_ERR_INVALID_ARG, "V must be < 2^18");
  if (k > kMaxK) return fail(PCT_ERR_UNSUPPORTED, "k exceeds %d", kMaxK);
  if ((U == nullptr) != (W == nullptr))
    return fail(PCT_ERR_INVALID_ARG, "U and W must both be given or NULL");
  if (!U && !L) return fail(PCT_ERR_INVALID_ARG, "need L or U/W");
  if (!parent_tok || !lse || !topk_tok || !topk_logp || !workspace ||
      (L && !parent_Lrow))
    return fail(PCT_ERR_INVALID_ARG, "required pointer is NULL");
  if (U && r < 1) return fail(PCT_ERR_INVALID_ARG, "r must be >= 1");
  if (uw_dtype != PCT_F32 && uw_dtype != PCT_BF16)
    return fail(PCT_ERR_INVALID_ARG, "unknown factor dtype");
  if (L && (L_row_stride < V || L_rows < 1))
    return fail(PCT_ERR_INVALID_ARG, "need L_row_stride >= V and L_rows >= 1");
  if (P > 65535)
    return fail(PCT_ERR_UNSUPPORTED, "P = %d exceeds 65535", P);
  if (workspace_bytes < pct_markov_logits_workspace(P, V, k))
    return fail(PCT_ERR_WORKSPACE, "workspace needs %zu bytes",
                pct_markov_logits_workspace(P, V, k));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool fac_aligned = U && aligned16(U) && aligned16(W);
  K1Plan pl = plan_k1(P, V, r, k, uw_dtype, U != nullptr, fac_aligned);
  Carve c{static_cast<char*>(workspace)};
  K1Args a{};
  a.part_c = c.take<float>((size_t)pl.n_slices * P);
  a.part_s = c.take<float>((size_t)pl.n_slices * P);
  // the candidate counters, then the tile queue: one clear for both
  a.gcnt = c.take<int32_t>(P + pl.n_tq);
  a.tq = pl.n_tq > 0 ? a.gcnt + P : nullptr;
  a.tiles_per_slice = pl.tiles_per_slice;
  a.gz = c.take<float>((size_t)pl.cap * P);
  a.gv = c.take<int32_t>((size_t)pl.cap * P);
  a.L = L;
  a.lstride = L ? L_row_stride : 0;
  a.L_rows = L ? L_rows : 1;
  a.vec_ok = L ? (aligned16(L) && L_row_stride % 4 == 0) : 1;
  a.U = U;
  a.W = W;
  a.dt = uw_dtype;
  a.V = V;
  a.r = r;
  a.P = P;
  a.k = k;
  a.ptok = parent_tok;
  a.plrow = L ? parent_Lrow : nullptr;
  a.theta = nullptr;
  a.n_tiles = pl.n_tiles;
  a.n_slices = pl.n_slices;
  a.vslice = pl.vslice;
  a.cap = pl.cap;
  a.z_out = z_out;
  hipError_t e = launch_fill_i32(a.gcnt, P + pl.n_tq, 0, s);
  if (e != hipSuccess) return hip_fail(e, "clear counters");
  {
    ProfScope ps(PROF_MARKOV, P, s);
    e = launch_k1(pl, a, s);
  }
  if (e != hipSuccess) return hip_fail(e, "markov kernel");
  {
    ProfScope ps(PROF_FINALIZE, P, s);
    e = launch_finalize(P, k, pl.n_slices, a.part_c, a.part_s, a.gcnt, a.gz,
                        a.gv, pl.cap, lse, topk_tok, topk_logp, s);
  }
  if (e != hipSuccess) return hip_fail(e, "finalize kernel");
  return PCT_OK;
}

// ------------------------------------------------------------------------
size_t pct_build_tree_workspace(const pct_tree_shape* shape) {
  if (check_shape(shape) != PCT_OK) return 0;
  TreePlan tp;
  if (plan_tree(shape, tp) != PCT_OK) return 0;
  TreeWs w;
  return carve_tree(shape, tp, nullptr, w);
}

pct_status pct_build_tree(const pct_tree_shape* shape, const float* L,
                          const void* U, const void* W,
                          const int32_t* anchor, int32_t* tok,
                          int32_t* parent, int32_t* depth, float* score,
                          int32_t* n_nodes, uint64_t* mask, void* workspace,
                          size_t workspace_bytes, void* stream) {
  pct_status st = check_shape(shape);
  if (st != PCT_OK) return st;
  if (!L || !anchor || !tok || !parent || !depth || !score || !n_nodes ||
      !workspace)
    return fail(PCT_ERR_INVALID_ARG, "required pointer is NULL");
  if ((U == nullptr) != (W == nullptr))
    return fail(PCT_ERR_INVALID_ARG, "U and W must both be given or NULL");
  pct_tree_shape sh = *shape;
  if (!U) sh.r = 0;
  else if (sh.r < 1)
    return fail(PCT_ERR_INVALID_ARG, "r must be >= 1 with Markov factors");
  // the MFMA operand loads, the packed U rows and the seed dot products
  // read the factors in 16-byte pieces
  if (U && (!aligned16(U) || !aligned16(W)))
    return fail(PCT_ERR_INVALID_ARG, "U and W must be 16-byte aligned");
  TreePlan tp;
  st = plan_tree(&sh, tp);
  if (st != PCT_OK) return st;
  TreeWs w;
  const size_t need = carve_tree(&sh, tp, nullptr, w);
  if (workspace_bytes < need)
    return fail(PCT_ERR_WORKSPACE, "workspace needs %zu bytes", need);
  carve_tree(&sh, tp, workspace, w);

  hipStream_t s = static_cast<hipStream_t>(stream);
  const int batch = sh.batch, B = sh.B, V = sh.V;
  const int64_t lstride = V;
  const int vec_ok = aligned16(L) && V % 4 == 0;
  const bool has_uw = U != nullptr;
  hipError_t e;

  // seeds: the best tokens of every L row
  {
    ProfScope ps(PROF_ROWTOP, (int64_t)batch * B, s);
    e = launch_rowtop(L, batch * B, V, lstride, vec_ok, w.rowtop, s);
  }
  if (e != hipSuccess) return hip_fail(e, "row top kernel");

  SeedArgs sa{};
  sa.L = L;
  sa.lstride = lstride;
  sa.rowtop = w.rowtop;
  sa.U = U;
  sa.W = W;
  sa.uw_bf16 = sh.uw_dtype == PCT_BF16;
  sa.r = sh.r;
  sa.V = V;
  sa.k = sh.k;
  sa.use_seed = sh.k <= kSeedT;
  // every depth of an MFMA plan reads its parents' U rows packed; init and
  // expand write them for the depth that follows
  sa.upack = tp.k1[1].kind == K1_MFMA ? w.upack : nullptr;

  Frontier f0{w.ftok[0], w.fpid[0], w.flrow[0], w.fs[0], w.ftheta[0]};
  Frontier f1{w.ftok[1], w.fpid[1], w.flrow[1], w.fs[1], w.ftheta[1]};
  {
    ProfScope ps(PROF_INIT, batch, s);
    e = launch_init(batch, B, anchor, f0, w.gcnt[1], w.tq, tp.max_tq, sa, s);
  }
  if (e != hipSuccess) return hip_fail(e, "init kernel");

  for (int d = 1; d <= B; ++d) {
    const Frontier& cur = (d & 1) ? f0 : f1;
    const Frontier& nxt = (d & 1) ? f1 : f0;
    const K1Plan& pl = tp.k1[d];
    const int Fp = tp.F[d - 1];
    const int P = has_uw ? batch * Fp : batch;
    K1Args a{};
    a.L = L;
    a.lstride = lstride;
    a.L_rows = (int64_t)batch * B;
    a.vec_ok = vec_ok;
    a.U = U;
    a.W = W;
    a.dt = sh.uw_dtype;
    a.V = V;
    a.r = sh.r;
    a.P = P;
    a.k = sh.k;
    if (has_uw) {
      a.ptok = cur.tok;
      // parent q*Fp + j reads row q*B + d-1: grouped rows
      a.plrow = nullptr;
      a.lrow_mul = B;
      a.lrow_add = d - 1;
      a.group_fp = Fp;
      a.lslots = vec_ok ? pl.lslots : 0;
      a.theta = sa.use_seed ? cur.theta : nullptr;
    } else {
      // no Markov term: every parent of request q shares row q*B + d-1, so
      // the statistics are computed once per request
      a.ptok = nullptr;
      a.plrow = nullptr;
      a.lrow_mul = B;
      a.lrow_add = d - 1;
      a.theta = nullptr;
    }
      a.n_tiles = pl.n_tiles;
    a.n_slices = pl.n_slices;
    a.vslice = pl.vslice;
    a.part_c = w.part_c;
    a.part_s = w.part_s;
    a.gcnt = w.gcnt[d & 1];
    a.gz = w.gz;
    a.gv = w.gv;
    a.cap = pl.cap;
    a.z_out = nullptr;
    a.upack = sa.upack;
    a.tq = pl.n_tq > 0 ? w.tq : nullptr;
    a.tiles_per_slice = pl.tiles_per_slice;
    {
      ProfScope ps(PROF_MARKOV, P, s);
      e = launch_k1(pl, a, s);
    }
    if (e != hipSuccess) return hip_fail(e, "markov kernel");

    ExpandArgs x{};
    x.d = d;
    x.B = B;
    x.Fp = Fp;
    x.Fn = tp.F[d];
    x.k = sh.k;
    x.N = sh.N;
    x.batch = batch;
    x.base_d = tp.base[d];
    x.pool_n = tp.pool_n;
    x.shared_stats = has_uw ? 0 : 1;
    x.n_slices = pl.n_slices;
    x.Pstat = P;
    x.cap = pl.cap;
    x.part_c = w.part_c;
    x.part_s = w.part_s;
    x.gcnt = a.gcnt;
    x.gz = w.gz;
    x.gv = w.gv;
    x.cur = cur;
    x.nxt = nxt;
    x.gcnt_next = (d < B) ? w.gcnt[(d + 1) & 1] : nullptr;
    x.pool_key = w.pool_key;
    x.seed = sa;
    x.seed.use_seed = has_uw && sa.use_seed;
    x.ckey = w.ckey;
    x.ppw = std::max(1, std::min(std::min(Fp, 32 / sh.k), 4));
    {
      ProfScope ps(PROF_EXPAND, batch, s);
      // the split form pays a second launch, which only the spread of at
      // least 64 parents over the chip recovers (batch-1 latency is better
      // with the single kernel)
      if (batch * Fp >= 64 && expand_split_ok(x)) {
        e = launch_merge(x, s);
        if (e == hipSuccess && d < B) e = launch_beam(x, s);
      } else {
        e = launch_expand(x, s);
      }
    }
    if (e != hipSuccess) return hip_fail(e, "expand kernel");
  }

  TopNArgs t{};
  t.batch = batch;
  t.B = B;
  t.N = sh.N;
  t.pool_n = tp.pool_n;
  for (int d = 1; d <= B + 1; ++d) t.base[d] = tp.base[d];  // base[66]
  t.pool_key = w.pool_key;
  t.tok = tok;
  t.parent = parent;
  t.depth = depth;
  t.score = score;
  t.n_nodes = n_nodes;
  {
    ProfScope ps(PROF_TOPN, batch, s);
    e = launch_topn(t, s);
  }
  if (e != hipSuccess) return hip_fail(e, "top-N kernel");
  if (mask) {
    {
      ProfScope ps(PROF_MASK, batch, s);
      e = launch_mask(batch, sh.N, parent, n_nodes, mask, s);
    }
    if (e != hipSuccess) return hip_fail(e, "mask kernel");
  }
  return PCT_OK;
}

// ------------------------------------------------------------------------
namespace {
pct_status check_cost(const pct_cost_model* cost) {
  if (!cost) return PCT_OK;
  if (!(cost->c1 >= 0.0) || !(cost->c2 >= 0.0) || !(cost->c_ell >= 0.0))
    return fail(PCT_ERR_INVALID_ARG,
                "cost model must be convex and increasing (c1, c2, c_ell "
                ">= 0)");
  if (!(cost->C_d + cost->c0 > 0.0))
    return fail(PCT_ERR_INVALID_ARG, "round cost at n = 0 must be > 0");
  return PCT_OK;
}

StopArgs stop_args(int N, const int32_t* n_avail, const float* score,
                   const int32_t* ctx_len, const pct_cost_model* cost) {
  StopArgs a{};
  a.N = N;
  a.n_avail = n_avail;
  a.score = score;
  a.ctx_len = cost ? ctx_len : nullptr;
  a.has_cost = cost != nullptr;
  if (cost) {
    a.C_d = cost->C_d;
    a.c0 = cost->c0;
    a.c1 = cost->c1;
    a.c2 = cost->c2;
    a.c_ell = cost->c_ell;
  }
  return a;
}
}  // namespace

namespace {
struct AdaptiveWs {
  float* lse_f;
  int32_t* ltok_f;
  float* llp_f;
  int32_t* flag;
  float* lse_s;
  int32_t* ltok_s;
  float* llp_s;
  // pieces of the single-read short-list pass
  float* pm;
  double* ps;
  float* cz;
  int32_t* cv;
};
size_t carve_adaptive(int batch, int B, int V, int n_max, void* ws,
                      AdaptiveWs& w, int& Kf, int& Ks) {
  const int64_t rows = (int64_t)batch * B;
  Kf = std::min(std::min(kAdaptiveShortList, n_max), V);
  Ks = std::min(n_max, V);
  Carve c{static_cast<char*>(ws)};
  w.lse_f = c.take<float>(rows);
  w.ltok_f = c.take<int32_t>(rows * Kf);
  w.llp_f = c.take<float>(rows * Kf);
  w.flag = c.take<int32_t>(batch);
  w.lse_s = c.take<float>(rows);
  w.ltok_s = c.take<int32_t>(rows * Ks);
  w.llp_s = c.take<float>(rows * Ks);
  const int64_t pieces = rows * rowpart_pieces(V);
  w.pm = c.take<float>(pieces);
  w.ps = c.take<double>(pieces);
  w.cz = c.take<float>(pieces * Kf);
  w.cv = c.take<int32_t>(pieces * Kf);
  return c.off;
}
pct_status check_adaptive(int32_t batch, int32_t B, int32_t V, int32_t n_max) {
  if (batch < 1 || B < 1 || V < 1 || n_max < 1)
    return fail(PCT_ERR_INVALID_ARG, "need batch, B, V, n_max >= 1");
  if (V >= (1 << 18)) return fail(PCT_ERR_INVALID_ARG, "V must be < 2^18");
  if (B > 255)
    return fail(PCT_ERR_UNSUPPORTED, "B = %d exceeds 255", B);
  if (n_max > kAdaptiveMaxNodes)
    return fail(PCT_ERR_UNSUPPORTED, "n_max = %d exceeds %d", n_max,
                kAdaptiveMaxNodes);
  return PCT_OK;
}
}  // namespace

size_t pct_build_tree_adaptive_workspace(int32_t batch, int32_t B, int32_t V,
                                         int32_t n_max) {
  if (check_adaptive(batch, B, V, n_max) != PCT_OK) return 0;
  AdaptiveWs w;
  int Kf, Ks;
  return carve_adaptive(batch, B, V, n_max, nullptr, w, Kf, Ks);
}

pct_status pct_build_tree_adaptive(int32_t batch, int32_t B, int32_t V,
                                   int32_t n_max, const float* L,
                                   const int32_t* ctx_len,
                                   const pct_cost_model* cost, int32_t* tok,
                                   int32_t* parent, int32_t* depth,
                                   float* score, int32_t* n_star, double* phi,
                                   double* throughput, uint64_t* mask,
                                   void* workspace, size_t workspace_bytes,
                                   void* stream) {
  pct_status st = check_adaptive(batch, B, V, n_max);
  if (st != PCT_OK) return st;
  if (!L || !tok || !parent || !depth || !score || !n_star || !phi ||
      !throughput || !workspace || (cost && !ctx_len))
    return fail(PCT_ERR_INVALID_ARG, "required pointer is NULL");
  st = check_cost(cost);
  if (st != PCT_OK) return st;
  AdaptiveWs w;
  int Kf, Ks;
  const size_t need = carve_adaptive(batch, B, V, n_max, nullptr, w, Kf, Ks);
  if (workspace_bytes < need)
    return fail(PCT_ERR_WORKSPACE, "workspace needs %zu bytes", need);
  carve_adaptive(batch, B, V, n_max, workspace, w, Kf, Ks);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int rows = batch * B;
  const int vec_ok = aligned16(L) && V % 4 == 0;
  double c5[5] = {0, 0, 0, 0, 0};
  if (cost) {
    c5[0] = cost->C_d;
    c5[1] = cost->c0;
    c5[2] = cost->c1;
    c5[3] = cost->c2;
    c5[4] = cost->c_ell;
  }
  const double* cp = cost ? c5 : nullptr;
  hipError_t e;
  {
    ProfScope ps(PROF_ROWSTATS, rows, s);
    if (rowpart_ok(V, Kf, vec_ok))
      e = launch_rowpart(L, rows, V, Kf, Kf, w.pm, w.ps, w.cz, w.cv, w.lse_f,
                         w.ltok_f, w.llp_f, s);
    else
      e = launch_rowsel(L, rows, V, B, Kf, Kf, nullptr, vec_ok, w.lse_f,
                        w.ltok_f, w.llp_f, s);
  }
  if (e != hipSuccess) return hip_fail(e, "row statistics kernel");
  const bool batched = bestfirst_batched_ok(B, V, n_max, Kf);
  {
    ProfScope ps(PROF_BESTFIRST, batch, s);
    e = launch_bestfirst(batch, B, V, n_max, Kf, Kf, Kf < V, w.ltok_f, w.llp_f,
                         ctx_len, cp, tok, parent, depth, score, n_star, phi,
                         throughput, w.flag, batched ? 2 : 0, s);
  }
  if (e != hipSuccess) return hip_fail(e, "best-first kernel");
  if (batched && Ks == Kf) {
    // requests the batched pass could not finish, on the same lists (they
    // are as long as the budget: every needed child rank is inside them)
    ProfScope ps(PROF_BESTFIRST, 0, s);
    e = launch_bestfirst(batch, B, V, n_max, Kf, Kf, Kf < V, w.ltok_f,
                         w.llp_f, ctx_len, cp, tok, parent, depth, score,
                         n_star, phi, throughput, w.flag, 1, s);
    if (e != hipSuccess) return hip_fail(e, "best-first kernel");
  }
  if (Ks > Kf) {
    // requests whose tree outgrew the short lists: full-length lists
    {
      ProfScope ps(PROF_ROWSTATS, 0, s);
      e = launch_rowsel(L, rows, V, B, Ks, Ks, w.flag, vec_ok, w.lse_s,
                        w.ltok_s, w.llp_s, s);
    }
    if (e != hipSuccess) return hip_fail(e, "row statistics kernel");
    {
      ProfScope ps(PROF_BESTFIRST, 0, s);
      e = launch_bestfirst(batch, B, V, n_max, Ks, Ks, Ks < V, w.ltok_s,
                           w.llp_s, ctx_len, cp, tok, parent, depth, score,
                           n_star, phi, throughput, w.flag, 1, s);
    }
    if (e != hipSuccess) return hip_fail(e, "best-first kernel");
  }
  if (mask) {
    ProfScope ps(PROF_MASK, batch, s);
    e = launch_mask(batch, n_max, parent, n_star, mask, s);
    if (e != hipSuccess) return hip_fail(e, "mask kernel");
  }
  return PCT_OK;
}

// ------------------------------------------------------------------------

size_t pct_build_tree_adaptive_pc_workspace(const pct_tree_shape* shape) {
  return pct_build_tree_workspace(shape);
}

pct_status pct_build_tree_adaptive_pc(
    const pct_tree_shape* shape, const float* L, const void* U,
    const void* W, const int32_t* anchor, const int32_t* ctx_len,
    const pct_cost_model* cost, int32_t* tok, int32_t* parent,
    int32_t* depth, float* score, int32_t* n_star, double* phi,
    double* throughput, uint64_t* mask, void* workspace,
    size_t workspace_bytes, void* stream) {
  pct_status st = check_cost(cost);
  if (st != PCT_OK) return st;
  if (!n_star || !phi || !throughput || (cost && !ctx_len))
    return fail(PCT_ERR_INVALID_ARG, "required pointer is NULL");
  // the tree in key order (a best-first order of its nodes); n_star holds
  // the node counts until the stop overwrites it
  st = pct_build_tree(shape, L, U, W, anchor, tok, parent, depth, score,
                      n_star, nullptr, workspace, workspace_bytes, stream);
  if (st != PCT_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  StopArgs a = stop_args(shape->N, n_star, score, ctx_len, cost);
  a.n_star = n_star;
  a.phi = phi;
  a.thr = throughput;
  a.tok = tok;
  a.parent = parent;
  a.depth = depth;
  a.score_out = score;
  hipError_t e;
  {
    ProfScope ps(PROF_STOP, shape->batch, s);
    e = launch_stop_scan(shape->batch, a, s);
  }
  if (e != hipSuccess) return hip_fail(e, "stop kernel");
  if (mask) {
    ProfScope ps(PROF_MASK, shape->batch, s);
    e = launch_mask(shape->batch, shape->N, parent, n_star, mask, s);
    if (e != hipSuccess) return hip_fail(e, "mask kernel");
  }
  return PCT_OK;
}

pct_status pct_throughput_curve(int32_t batch, int32_t N, const float* score,
                                const int32_t* n_nodes,
                                const int32_t* ctx_len,
                                const pct_cost_model* cost, double* f,
                                void* stream) {
  if (batch < 1 || N < 1)
    return fail(PCT_ERR_INVALID_ARG, "need batch, N >= 1");
  if (!score || !n_nodes || !f || (cost && !ctx_len))
    return fail(PCT_ERR_INVALID_ARG, "required pointer is NULL");
  pct_status st = check_cost(cost);
  if (st != PCT_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  StopArgs a = stop_args(N, n_nodes, score, ctx_len, cost);
  a.f = f;
  hipError_t e;
  {
    ProfScope ps(PROF_STOP, batch, s);
    e = launch_stop_scan(batch, a, s);
  }
  if (e != hipSuccess) return hip_fail(e, "throughput curve kernel");
  return PCT_OK;
}

// ------------------------------------------------------------------------
pct_status pct_tree_mask(int32_t batch, int32_t N, const int32_t* parent,
                         const int32_t* n_nodes, uint64_t* mask,
                         void* stream) {
  if (batch < 1 || N < 1) return fail(PCT_ERR_INVALID_ARG, "batch, N >= 1");
  if (!parent || !n_nodes || !mask)
    return fail(PCT_ERR_INVALID_ARG, "required pointer is NULL");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  {
    ProfScope ps(PROF_MASK, batch, s);
    e = launch_mask(batch, N, parent, n_nodes, mask, s);
  }
  if (e != hipSuccess) return hip_fail(e, "mask kernel");
  return PCT_OK;
}

pct_status pct_verify_accept(int32_t batch, int32_t N, int32_t B,
                             const int32_t* tok, const int32_t* parent,
                             const int32_t* depth, const int32_t* n_nodes,
                             const uint64_t* mask, const int32_t* target,
                             int32_t* tau, int32_t* accept_node,
                             int32_t* accept_tok, void* stream) {
  if (batch < 1 || N < 1 || B < 1 || N > 8192)
    return fail(PCT_ERR_INVALID_ARG, "need batch, B >= 1 and 1 <= N <= 8192");
  if (!tok || !parent || !depth || !n_nodes || !target || !tau ||
      !accept_node || !accept_tok)
    return fail(PCT_ERR_INVALID_ARG, "required pointer is NULL");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  {
    ProfScope ps(PROF_ACCEPT, batch, s);
    e = launch_accept(batch, N, B, tok, parent, depth, n_nodes, mask, target,
                      tau, accept_node, accept_tok, s);
  }
  if (e != hipSuccess) return hip_fail(e, "accept kernel");
  return PCT_OK;
}

namespace {
pct_status check_sample(int32_t batch, int32_t N, int32_t B, int32_t V) {
  if (batch < 1 || N < 1 || B < 1 || N > 8192 || V < 1)
    return fail(PCT_ERR_INVALID_ARG,
                "need batch, B, V >= 1 and 1 <= N <= 8192");
  if (batch > 65535)
    return fail(PCT_ERR_UNSUPPORTED, "batch = %d exceeds 65535", batch);
  return PCT_OK;
}
}  // namespace

size_t pct_verify_sample_workspace(int32_t batch, int32_t N, int32_t V) {
  if (batch < 1 || N < 1 || N > 8192 || V < 1 || batch > 65535) return 0;
  return sample_workspace((int64_t)batch * (N + 1), V);
}

pct_status pct_verify_sample(int32_t batch, int32_t N, int32_t B, int32_t V,
                             const int32_t* tok, const int32_t* parent,
                             const int32_t* depth, const int32_t* n_nodes,
                             const uint64_t* mask, const float* target_logits,
                             double temperature, uint64_t seed,
                             int32_t* sampled, int32_t* tau,
                             int32_t* accept_node, int32_t* accept_tok,
                             void* workspace, size_t workspace_bytes,
                             void* stream) {
  pct_status st = check_sample(batch, N, B, V);
  if (st != PCT_OK) return st;
  if (!(temperature > 0.0) || !(temperature < 1e300))
    return fail(PCT_ERR_INVALID_ARG, "temperature must be positive and finite");
  if (!tok || !parent || !depth || !n_nodes || !target_logits || !sampled ||
      !tau || !accept_node || !accept_tok)
    return fail(PCT_ERR_INVALID_ARG, "required pointer is NULL");
  const size_t need = sample_workspace((int64_t)batch * (N + 1), V);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(PCT_ERR_WORKSPACE, "workspace needs %zu bytes", need);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  {
    ProfScope ps(PROF_SAMPLE, batch, s);
    e = launch_sample(batch, N + 1, V, target_logits, 1.0 / temperature,
                      seed, n_nodes, sampled, workspace, s);
  }
  if (e != hipSuccess) return hip_fail(e, "sample kernel");
  {
    ProfScope ps(PROF_ACCEPT, batch, s);
    e = launch_accept(batch, N, B, tok, parent, depth, n_nodes, mask, sampled,
                      tau, accept_node, accept_tok, s);
  }
  if (e != hipSuccess) return hip_fail(e, "accept kernel");
  return PCT_OK;
}

}  // extern "C"
