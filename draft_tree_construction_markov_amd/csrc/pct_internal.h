// pct_internal.h -- host-side plumbing shared by the libpctree translation
// units: kernel argument blocks, launch plans and launcher declarations.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pct {

// Candidate-list entry of the fused Markov kernel.
struct ZV {
  float z;
  int32_t v;
};

// Arguments of the fused Markov / log-sum-exp / top-k kernels.
struct K1Args {
  const float* L;      // logits rows (may be null: z = Markov only)
  int64_t lstride;     // elements between L rows
  int vec_ok;          // rows 16-byte aligned: vector loads allowed
  const void* U;       // [V][r] factors (null: z = L)
  const void* W;       // [V][r], vocab-major
  int dt;              // factor element type: 0 fp32, 1 bf16
  int V, r, P, k;
  const int32_t* ptok;   // [P] parent tokens
  const int32_t* plrow;  // [P] L row of each parent (null: p*lrow_mul+lrow_add)
  int lrow_mul, lrow_add;
  int64_t L_rows;        // rows of L (row indices are clamped to it)
  // Grouped rows: when group_fp > 0 and plrow is null, parent p reads row
  // (p / group_fp) * lrow_mul + lrow_add, and the fused kernel stages the
  // workgroup's distinct rows of each vocabulary tile through LDS
  // (lslots row slots per buffer).
  int group_fp, lslots;
  const float* theta;    // [P] candidate threshold seeds (null: -inf)
  int n_tiles, n_slices;  // mfma: 64-vocab tiles; workgroups per parent tile
  int tiles_per_slice;    // mfma without a tile queue: contiguous tiles each
  int vslice;                              // simple: vocab per slice
  float* part_c;   // [n_slices][P] running max in log2 units
  float* part_s;   // [n_slices][P] sum of 2^(z*log2e - part_c)
  int32_t* gcnt;   // [P] candidates per parent (zeroed before launch)
  float* gz;       // [P][cap]
  int32_t* gv;     // [P][cap]
  int cap;
  float* z_out;    // [P][V] optional
  // U rows of the parents in MFMA operand order (null: gathered from U):
  // 16-byte chunk c of parent p's row at ((p/32) * r/16 + c/2) * 64 +
  // (c%2) * 32 + p%32
  const uint4* upack;
  // Tile queue of the tiled MFMA kernel, two counters per parent tile
  // (grid row): tickets handed out, workgroups finished.  Both are zero
  // before a launch and the launch's last workgroup zeroes them again.
  // Null: every workgroup takes its slice of contiguous tiles.
  int32_t* tq;
};

enum K1Kind { K1_MFMA = 0, K1_SIMPLE = 1 };

struct K1Plan {
  int kind;
  int thin;  // MFMA, at most 32 parents: markov_topk_thin (vslice rows)
  int NB, NW, R16;
  int lslots;  // LDS row slots for grouped rows (0: rows read directly)
  int n_tiles, tiles_per_slice, n_slices, vslice;
  int n_tq;  // tile-queue counters the launch needs (0: contiguous slices)
  int cap;  // candidate capacity per parent
  size_t lds;        // dynamic LDS bytes of the launch
  size_t lds_total;  // static + dynamic, for occupancy planning
  dim3 grid, block;
};

constexpr int kSeedT = 32;         // top tokens of each L row used for seeds
constexpr int kLdsRowSlots = 36;   // staged L rows per buffer (fused kernel)
constexpr int kSmallRowSlots = 16; // the same, beside long top-k lists
constexpr int kSimpleThreads = 128;
constexpr int kMaxPool = 8192;     // generated children per request
constexpr int kMaxCand = 2048;     // children per request and depth
constexpr int kMaxK = 64;

// Allow a kernel more than the default 64 KB of dynamic LDS; only called
// when a launch needs it.  A failure is consumed (not left as the thread's
// last error) and returned.
inline hipError_t allow_lds(const void* fn, size_t bytes) {
  if (bytes <= 64 * 1024) return hipSuccess;
  hipError_t e = hipFuncSetAttribute(
      fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e != hipSuccess) (void)hipGetLastError();
  return e;
}

// Kernel kinds reported by the profiler (see pct_profile_read).
enum ProfKind {
  PROF_MARKOV = 0,   // fused Markov / log-sum-exp / top-k kernel
  PROF_EXPAND = 1,   // per-request merge, scores and beam
  PROF_TOPN = 2,     // global top-N
  PROF_MASK = 3,     // ancestry mask
  PROF_ACCEPT = 4,   // acceptance walk
  PROF_ROWTOP = 5,   // seed pre-pass over the logit rows
  PROF_INIT = 6,     // depth-1 frontier
  PROF_ROWSTATS = 7, // adaptive: streaming log-softmax + select
  PROF_BESTFIRST = 8,// adaptive: best-first order + stop
  PROF_FINALIZE = 9, // standalone Markov call: per-parent results
  PROF_STOP = 10,    // throughput stop / curve scan
  PROF_SAMPLE = 11   // sampled target tokens
};

// RAII bracket of one launch (no-op unless profiling is enabled).
class ProfScope {
 public:
  ProfScope(int kind, int64_t units, hipStream_t s);
  ~ProfScope();

 private:
  hipStream_t stream_;
  int idx_;
};

// Sets the calling thread's pct_last_error() text and returns st.
}  // namespace pct
#include "../../include/pctree.h"
namespace pct {
pct_status set_error(pct_status st, const char* msg);

K1Plan plan_k1(int P, int V, int r, int k, int uw_dtype, bool has_uw,
               bool allow_mfma = true, int group_fp = 0);
hipError_t launch_k1(const K1Plan& pl, const K1Args& a, hipStream_t s);

// Per-request state of the depth loop.
struct Frontier {
  int32_t* tok;
  int32_t* pid;
  int32_t* lrow;
  float* s;
  float* theta;
};

struct SeedArgs {
  const float* L;
  int64_t lstride;
  const int32_t* rowtop;  // [rows][kSeedT]
  const void* U;
  const void* W;
  int uw_bf16, r, V, k;
  int use_seed;
  uint4* upack;  // packed U rows of the next parents (null: not written)
};

// Index of 16-byte chunk c (of 2*R16 per row) of parent p in the packed U
// layout read by the fused kernel: one 64-lane MFMA operand load per
// (32-parent block, rank step) covers 1 KB of consecutive memory.
__host__ __device__ inline int64_t upack_index(int p, int c, int R16) {
  return ((int64_t)(p >> 5) * R16 + (c >> 1)) * 64 + (c & 1) * 32 + (p & 31);
}

struct ExpandArgs {
  int d, B, Fp, Fn, k, N, batch;
  int base_d, pool_n;
  int shared_stats;  // all parents of a request share one statistics row
  int n_slices, Pstat, cap;
  const float* part_c;
  const float* part_s;
  const int32_t* gcnt;
  const float* gz;
  const int32_t* gv;
  Frontier cur, nxt;
  int32_t* gcnt_next;  // zeroed for the next depth's parents
  uint64_t* pool_key;  // [batch][pool_n]
  SeedArgs seed;
  // split form (merge_kernel + beam_kernel) only
  uint64_t* ckey;  // [batch][Fp*k] this depth's child keys
  int ppw;         // parents per merge workgroup (ppw <= 4, ppw * k <= 32)
};

struct TopNArgs {
  int batch, B, N, pool_n;
  int base[66];  // pool id where depth d starts (d = 1..B), base[B+1] = end
  const uint64_t* pool_key;
  int32_t *tok, *parent, *depth;
  float* score;
  int32_t* n_nodes;
};

hipError_t launch_rowtop(const float* L, int rows, int V, int64_t lstride,
                         int vec_ok, int32_t* rowtop, hipStream_t s);
hipError_t launch_init(int batch, int B, const int32_t* anchor, Frontier f,
                       int32_t* gcnt, int32_t* tq, int n_tq,
                       const SeedArgs& sa, hipStream_t s);
hipError_t launch_expand(const ExpandArgs& a, hipStream_t s);
// the split form applies to bf16 factors with seeds by MFMA, staged
// partials and one statistics row per parent
bool expand_split_ok(const ExpandArgs& a);
hipError_t launch_merge(const ExpandArgs& a, hipStream_t s);
hipError_t launch_beam(const ExpandArgs& a, hipStream_t s);
hipError_t launch_topn(const TopNArgs& a, hipStream_t s);
hipError_t launch_finalize(int P, int k, int n_slices, const float* part_c,
                           const float* part_s, const int32_t* gcnt,
                           const float* gz, const int32_t* gv, int cap,
                           float* lse, int32_t* topk_tok, float* topk_logp,
                           hipStream_t s);
hipError_t launch_rowsel(const float* L, int rows, int V, int B, int K,
                         int kstride, const int32_t* only_flagged, int vec_ok,
                         float* lse, int32_t* ltok, float* llp, hipStream_t s);
hipError_t launch_bestfirst(int batch, int B, int V, int n_max, int klist,
                            int kstride, int truncated, const int32_t* ltok,
                            const float* llp, const int32_t* ctx_len,
                            const double* cost5, int32_t* tok,
                            int32_t* parent, int32_t* depth, float* score,
                            int32_t* n_star, double* phi, double* thr,
                            int32_t* flag, int slow, hipStream_t s);
// slow: 0 serial first pass (flags requests that outgrow the lists),
// 1 serial pass over the flagged requests, 2 batched first pass (flags the
// same requests and those whose enumeration overflows), usable when
// bestfirst_batched_ok()
bool bestfirst_batched_ok(int B, int V, int n_max, int klist);
constexpr int kAdaptiveShortList = 64;  // list length of the first pass
constexpr int kAdaptiveMaxNodes = 1024;
// single-read row statistics: lists up to kPartMaxK, rows cut into at most
// kPartMaxParts register-resident pieces
constexpr int kPartMaxK = 128;
constexpr int kPartMaxParts = 8;
int rowpart_pieces(int V);
bool rowpart_ok(int V, int K, int vec_ok);
hipError_t launch_rowpart(const float* L, int rows, int V, int K, int kstride,
                          float* pm, double* ps, float* cz, int32_t* cv,
                          float* lse, int32_t* ltok, float* llp,
                          hipStream_t s);
hipError_t launch_fill_i32(int32_t* p, int n, int32_t v, hipStream_t s);

// Throughput stop / curve over best-first-ordered trees (one wave per
// request).  Pointers that are null are not written.
struct StopArgs {
  int N;                   // row stride of the ordered lists
  const int32_t* n_avail;  // [batch] nodes in each list (may alias n_star)
  const float* score;      // [batch][N] scores in best-first order
  const int32_t* ctx_len;  // [batch] or null (no cost model)
  int has_cost;
  double C_d, c0, c1, c2, c_ell;
  int32_t* n_star;  // [batch]
  double* phi;      // [batch] Phi(n*)
  double* thr;      // [batch] (1 + Phi(n*)) / D(n*)
  double* f;        // [batch][N+1] f(n) = (1 + Phi_n) / D(n)
  // pads written past n* (tok -1, parent -1, depth 0, score -inf)
  int32_t *tok, *parent, *depth;
  float* score_out;
};
hipError_t launch_stop_scan(int batch, const StopArgs& a, hipStream_t s);
hipError_t launch_mask(int batch, int N, const int32_t* parent,
                       const int32_t* n_nodes, uint64_t* mask, hipStream_t s);
// sampled target tokens: each row is cut into sample_slices(rows, V)
// slices; with more than one, sample_workspace(rows, V) bytes of partial
// results are merged by a second kernel
int sample_slices(int64_t rows, int V);
size_t sample_workspace(int64_t rows, int V);
hipError_t launch_sample(int batch, int N1, int V, const float* logits,
                         double inv_t, uint64_t seed, const int32_t* n_nodes,
                         int32_t* sampled, void* ws, hipStream_t s);
hipError_t launch_accept(int batch, int N, int B, const int32_t* tok,
                         const int32_t* parent, const int32_t* depth,
                         const int32_t* n_nodes, const uint64_t* mask,
                         const int32_t* target, int32_t* tau,
                         int32_t* accept_node, int32_t* accept_tok,
                         hipStream_t s);

}  // namespace pct
