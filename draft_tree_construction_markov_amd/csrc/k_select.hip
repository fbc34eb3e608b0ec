// k_select.hip -- per-request selection kernels of the parent-conditioned
// tree (PCTree article, "straight draft"): merging the per-slice partials of
// the fused Markov kernel into each parent's log-normaliser and local top-k,
// path scores s(c) = s(p) + log pi(c|p), the per-depth beam (top-k pruning
// at each stage), and the global top-N that fits the verify budget.  Also
// the threshold seeds that let the fused kernel skip almost every logit.
#include "pct_device.h"
#include "pct_internal.h"

#include <algorithm>

namespace pct {



// ---------------------------------------------------------------------
// Seeds.  For a parent p, theta_p = (k-th largest z over a small token
// subset) - margin is a lower bound of the k-th largest z over the whole
// row, so every true top-k logit passes "z >= theta_p" in the fused kernel.
// The subset is the kSeedT best tokens of the parent's L row.  The margin
// covers the difference between this kernel's fp32 dot product and the
// MFMA's fp32 accumulation of the same exact bf16 products:
// |dM| <= 2 r 2^-24 sum|u w| (each side's recursive-sum bound; doubled
// again for safety) plus a few ulps of |z| for the final fp32 adds.

// Per L row, kSeedT tokens of large L.  The row is cut into kRowTopPieces
// pieces with one workgroup each (enough workgroups to keep every CU
// streaming); each thread keeps its best element of the piece and the piece
// contributes the kSeedT / kRowTopPieces best of those.  Any subset is a
// valid seed; this one is close to the row's top kSeedT.
constexpr int kRowTopPieces = 8;
constexpr int kRowTopVec = 19;  // 16-byte loads per thread and round
constexpr int kRowTopSlots = kSeedT / kRowTopPieces;

__global__ __launch_bounds__(256) void row_top_kernel(const float* L, int V,
                                                       int64_t lstride,
                                                       int vec_ok,
                                                       int32_t* rowtop) {
  __shared__ __align__(16) float sz[256];
  __shared__ __align__(16) int32_t sv[256];
  __shared__ __align__(16) float cz[256 + 4];
  __shared__ __align__(16) int32_t cv[256 + 4];
  __shared__ float tau_z;
  __shared__ int32_t tau_v;
  __shared__ int wcount[4];
  const int row = blockIdx.x, piece = blockIdx.y, tid = threadIdx.x;
  const float* Lr = L + (int64_t)row * lstride;
  // piece bounds in tokens, a multiple of 4 apart so that vectors align
  const int span = ((V + 4 * kRowTopPieces - 1) / (4 * kRowTopPieces)) * 4;
  const int v0 = min(piece * span, V), v1 = min(v0 + span, V);
  float bz = neg_inf();
  int32_t bv = 0x7fffffff;
  // Within a thread the tokens only grow, so a strict comparison keeps the
  // smallest token among equal logits: a max and a select per element.
  auto see = [&](float z, int v) __attribute__((always_inline)) {
    const bool b = z > bz;
    bz = b ? z : bz;
    bv = b ? v : bv;
  };
  if (vec_ok) {
    const float4* L4 = reinterpret_cast<const float4*>(Lr);
    const int i0b = v0 / 4, i1 = v1 / 4;  // whole vectors; V % 4 == 0 here
    // kRowTopVec independent 16-byte loads in flight per thread (a whole
    // piece of a 151936-token row in one round); out-of-range slots reload
    // the first vector of the piece and are masked to -inf.  Non-temporal:
    // the rows are read once here, and the factor matrix W, which every
    // depth reads again, stays in the caches.
    for (int i0 = i0b + tid; i0 < i1; i0 += kRowTopVec * 256) {
      float4 x[kRowTopVec];
#pragma unroll
      for (int u = 0; u < kRowTopVec; ++u) {
        const int i = i0 + u * 256;
        const f32x4 y = __builtin_nontemporal_load(
            reinterpret_cast<const f32x4*>(L4 + (i < i1 ? i : i0b)));
        x[u] = make_float4(y.x, y.y, y.z, y.w);
      }
#pragma unroll
      for (int u = 0; u < kRowTopVec; ++u) {
        const int i = i0 + u * 256;
        const bool in = i < i1;
        const int v = 4 * i;
        see(in ? x[u].x : neg_inf(), v);
        see(in ? x[u].y : neg_inf(), v + 1);
        see(in ? x[u].z : neg_inf(), v + 2);
        see(in ? x[u].w : neg_inf(), v + 3);
      }
    }
  } else {
    for (int v = v0 + tid; v < v1; v += 256) see(Lr[v], v);
  }
  sz[tid] = bz;
  sv[tid] = bv;
  // slots without a distinct token (tiny pieces) stay -1 and are skipped
  int32_t* out = rowtop + (int64_t)row * kSeedT + piece * kRowTopSlots;
  if (tid < kRowTopSlots) out[tid] = -1;
  if (tid == 0) {
    tau_z = neg_inf();
    tau_v = 0x7fffffff;
  }
  __syncthreads();
  // The slots take the kRowTopSlots first of the 256 thread bests in
  // (logit desc, token asc) order.  The kRowTopSlots-th of wave 0's 64
  // entries is at or after the kRowTopSlots-th of all 256, so only entries
  // at or before it can place; every entry before a candidate is itself a
  // candidate, so a candidate's rank among the candidates is its rank among
  // all.  (If wave 0 has fewer distinct entries, every entry is a
  // candidate.)
  const float4* z4 = reinterpret_cast<const float4*>(sz);
  const int4* v4 = reinterpret_cast<const int4*>(sv);
  if (tid < 64) {
    int r0 = 0;
#pragma unroll 4
    for (int j = 0; j < 16; ++j) {
      const float4 z = z4[j];
      const int4 v = v4[j];
      r0 += zv_before(z.x, v.x, bz, bv) + zv_before(z.y, v.y, bz, bv) +
            zv_before(z.z, v.z, bz, bv) + zv_before(z.w, v.w, bz, bv);
    }
    if (r0 == kRowTopSlots - 1) {  // equal entries carry equal values
      tau_z = bz;
      tau_v = bv;
    }
  }
  __syncthreads();
  const bool cand = !zv_before(tau_z, tau_v, bz, bv);
  const uint64_t bal = __ballot(cand);
  const int lane = tid & 63, wave = tid >> 6;
  if (lane == 0) wcount[wave] = __popcll(bal);
  __syncthreads();
  int off = 0, m = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    off += w < wave ? wcount[w] : 0;
    m += wcount[w];
  }
  if (cand) {
    const int at = off + __popcll(bal & ((1ull << lane) - 1));
    cz[at] = bz;
    cv[at] = bv;
  }
  // pad to whole vectors with entries that come before nothing
  if (tid < 4 && m + tid < 256 + 4) {
    cz[m + tid] = neg_inf();
    cv[m + tid] = 0x7fffffff;
  }
  __syncthreads();
  if (cand) {
    int rank = 0;
    const float4* c4 = reinterpret_cast<const float4*>(cz);
    const int4* d4 = reinterpret_cast<const int4*>(cv);
    for (int j = 0; j < (m + 3) / 4; ++j) {
      const float4 z = c4[j];
      const int4 v = d4[j];
      rank += zv_before(z.x, v.x, bz, bv) + zv_before(z.y, v.y, bz, bv) +
              zv_before(z.z, v.z, bz, bv) + zv_before(z.w, v.w, bz, bv);
    }
    if (rank < kRowTopSlots && bv < V) out[rank] = bv;
  }
}

__device__ __forceinline__ float dot_bf16(const uint16_t* u, const uint16_t* w,
                                          int r, float& absacc) {
  float acc = 0.f, aa = 0.f;
  if ((r & 7) == 0) {
    const uint4* u4 = reinterpret_cast<const uint4*>(u);
    const uint4* w4 = reinterpret_cast<const uint4*>(w);
    for (int c = 0; c < r / 8; ++c) {
      const uint4 a = u4[c], b = w4[c];
      const uint32_t ua[4] = {a.x, a.y, a.z, a.w};
      const uint32_t wb[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float u0 = __uint_as_float(ua[i] << 16);
        const float u1 = __uint_as_float(ua[i] & 0xffff0000u);
        const float w0 = __uint_as_float(wb[i] << 16);
        const float w1 = __uint_as_float(wb[i] & 0xffff0000u);
        acc = fmaf(u0, w0, acc);
        aa += fabsf(u0 * w0);
        acc = fmaf(u1, w1, acc);
        aa += fabsf(u1 * w1);
      }
    }
  } else {
    for (int j = 0; j < r; ++j) {
      const float p = bf16_bits_to_float(u[j]) * bf16_bits_to_float(w[j]);
      acc = fmaf(bf16_bits_to_float(u[j]), bf16_bits_to_float(w[j]), acc);
      aa += fabsf(p);
    }
  }
  absacc = aa;
  return acc;
}

__device__ __forceinline__ float dot_f32(const float* u, const float* w,
                                         int r, float& absacc) {
  float acc = 0.f, aa = 0.f;
  for (int j = 0; j < r; ++j) {
    acc = fmaf(u[j], w[j], acc);
    aa += fabsf(u[j] * w[j]);
  }
  absacc = aa;
  return acc;
}

// One wave: the seed threshold of a parent with token ptok whose logits are
// L row `row`.
__device__ float seed_theta(const SeedArgs& sa, int ptok, int row, int lane) {
  if (!sa.use_seed || sa.k > kSeedT) return neg_inf();
  const float* Lr = sa.L + (int64_t)row * sa.lstride;
  float z = neg_inf(), A = 0.f;
  ptok = min(max(ptok, 0), sa.V - 1);
  const int v = lane < kSeedT ? sa.rowtop[(int64_t)row * kSeedT + lane] : -1;
  if (v >= 0 && v < sa.V) {
    float m = 0.f;
    if (sa.U) {
      if (sa.uw_bf16)
        m = dot_bf16(reinterpret_cast<const uint16_t*>(sa.U) +
                         (int64_t)ptok * sa.r,
                     reinterpret_cast<const uint16_t*>(sa.W) +
                         (int64_t)v * sa.r,
                     sa.r, A);
      else
        m = dot_f32(reinterpret_cast<const float*>(sa.U) + (int64_t)ptok * sa.r,
                    reinterpret_cast<const float*>(sa.W) + (int64_t)v * sa.r,
                    sa.r, A);
    }
    z = Lr[v] + m;
  }
  // rank of each lane's z (ties by lane index)
  int rank = 0;
  for (int o = 0; o < kSeedT; ++o) {
    const float zo = __shfl(z, o, kWave);
    rank += (zo > z) || (zo == z && o < lane);
  }
  float kth = (lane < kSeedT && rank == sa.k - 1) ? z : neg_inf();
  kth = wave_max(kth);
  const float zmax = wave_max(z != neg_inf() ? fabsf(z) : 0.f);
  const float Amax = wave_max(A);
  const float margin = 4.f * (float)sa.r * 5.9604645e-8f * Amax +
                       4.f * 1.1920929e-7f * zmax + 1e-30f;
  return kth - margin;
}

// ---------------------------------------------------------------------
// Merging the fused kernel's partials (one wave per parent).

// log-normaliser from [S][P] partials (c in log2 units, s = sum 2^(.-c)),
// in one pass over memory: each lane keeps a running (max, sum) with fp32
// scale factors and a double sum; lanes combine by shuffles.
__device__ float wave_merge_lse(const float* part_c, const float* part_s,
                                int S, int P, int p, int lane) {
  float cm = neg_inf();
  double acc = 0.0;
  for (int s0 = 0; s0 < S; s0 += 4 * kWave) {
    float c[4], v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s = s0 + i * kWave + lane;
      c[i] = s < S ? part_c[(int64_t)s * P + p] : neg_inf();
      v[i] = s < S ? part_s[(int64_t)s * P + p] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (c[i] == neg_inf() || !(v[i] > 0.f)) continue;
      if (c[i] > cm) {
        acc = acc * (double)__builtin_amdgcn_exp2f(cm - c[i]) + (double)v[i];
        cm = c[i];
      } else {
        acc += (double)v[i] * (double)__builtin_amdgcn_exp2f(c[i] - cm);
      }
    }
  }
  const float gm = wave_max(cm);
  acc = (cm == neg_inf()) ? 0.0
                          : acc * (double)__builtin_amdgcn_exp2f(cm - gm);
  acc = wave_sum(acc);
  return (float)(kLn2 * ((double)gm + log2(acc)));
}

// The i-th best candidate (z desc, token asc) of a parent, i = 0..k-1, by k
// passes that each take the best entry after the previous pick.  Results on
// every lane.
template <typename F>
__device__ void wave_topk(const float* gz, const int32_t* gv, int cnt, int k,
                          int lane, F&& emit) {
  float pz = pos_inf();
  int32_t pv = -1;
  if (cnt <= kWave) {
    // one candidate per lane, loaded once
    const float cz = lane < cnt ? gz[lane] : neg_inf();
    const int32_t cv = lane < cnt ? gv[lane] : 0x7fffffff;
    for (int i = 0; i < k; ++i) {
      float bz = neg_inf();
      int32_t bv = 0x7fffffff;
      if (zv_before(pz, pv, cz, cv)) {
        bz = cz;
        bv = cv;
      }
      wave_best_zv(bz, bv);
      if (bv == 0x7fffffff) bv = 0;  // fewer than k candidates: cannot
      emit(i, bz, bv);                // happen with a valid seed
      pz = bz;
      pv = bv;
    }
    return;
  }
  for (int i = 0; i < k; ++i) {
    float bz = neg_inf();
    int32_t bv = 0x7fffffff;
    for (int e = lane; e < cnt; e += kWave) {
      const float z = gz[e];
      const int32_t v = gv[e];
      if (zv_before(pz, pv, z, v) && zv_before(z, v, bz, bv)) {
        bz = z;
        bv = v;
      }
    }
    wave_best_zv(bz, bv);
    if (bv == 0x7fffffff) bv = 0;
    emit(i, bz, bv);
    pz = bz;
    pv = bv;
  }
}

// The k best candidates (z desc, token asc) of a parent, one wave: with at
// most 64 candidates every lane takes one and counts the candidates that
// come before it (read back from the wave's LDS scratch, 64 float2), so the
// k results come out in one pass; emit(i, z, v) is called by the lane that
// holds result i.  Missing results (fewer than k candidates, which a valid
// seed rules out) are emitted by lane 0 as (-inf, 0).  More than 64
// candidates take k passes of wave-wide arg-max.
template <typename F>
__device__ void wave_topk_rank(const float* gz, const int32_t* gv, int cnt,
                               int k, int lane, float2* scratch, F&& emit,
                               bool have = false, float hz = 0.f,
                               int32_t hv = 0) {
  if (cnt > kWave) {
    wave_topk(gz, gv, cnt, k, lane, [&](int i, float z, int32_t v) {
      if (lane == 0) emit(i, z, v);
    });
    return;
  }
  // (hz, hv): this lane's slot, already loaded by the caller when `have`
  const float cz = lane < cnt ? (have ? hz : gz[lane]) : neg_inf();
  const int32_t cv = lane < cnt ? (have ? hv : gv[lane]) : 0x7fffffff;
  scratch[lane] = make_float2(cz, __int_as_float(cv));
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  int rank = 0;
  for (int o = 0; o < cnt; ++o) {
    const float2 e = scratch[o];
    rank += zv_before(e.x, __float_as_int(e.y), cz, cv);
  }
  if (lane < cnt && rank < k) emit(rank, cz, cv);
  if (lane == 0)
    for (int i = cnt; i < k; ++i) emit(i, neg_inf(), 0);
}

// Seeds of up to 32 parents that share one L row (one wave), computed with
// the same bf16 MFMA as the fused kernel: the seed tokens form the 32 "vocab"
// rows of a 32x32x16 block and the parents its columns.  A second MFMA on
// |U|, |W| gives sum|u w| for the rounding margin.  Operands come from LDS
// (staged by the caller): wrows[32][cs] and urows[32][cs] 16-byte chunks
// (cs = r/8 + 1, one chunk of padding), lval[32] the seed tokens' logits,
// vt[32] the seed tokens (-1 = none).  Returns the threshold of the parent
// in column lane%32 (meaningful for columns < npar).
__device__ float seed_theta_mfma(const SeedArgs& sa, const uint4* wrows,
                                 const uint4* urows, const float* lval,
                                 const int* vt, int lane) {
  const int h = lane >> 5, col = lane & 31;
  const int cs = sa.r / 8 + 1;
  f32x16 acc, aacc;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    acc[j] = 0.f;
    aacc[j] = 0.f;
  }
  for (int kk = 0; kk < sa.r / 16; ++kk) {
    const uint4 w4 = wrows[col * cs + 2 * kk + h];
    const uint4 u4 = urows[col * cs + 2 * kk + h];
    const uint4 wa = make_uint4(w4.x & 0x7fff7fffu, w4.y & 0x7fff7fffu,
                                w4.z & 0x7fff7fffu, w4.w & 0x7fff7fffu);
    const uint4 ua = make_uint4(u4.x & 0x7fff7fffu, u4.y & 0x7fff7fffu,
                                u4.z & 0x7fff7fffu, u4.w & 0x7fff7fffu);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
        __builtin_bit_cast(bf16x8, w4), __builtin_bit_cast(bf16x8, u4), acc,
        0, 0, 0);
    aacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
        __builtin_bit_cast(bf16x8, wa), __builtin_bit_cast(bf16x8, ua), aacc,
        0, 0, 0);
  }
  // register j holds seed token 8*(j/4) + 4h + j%4 of this column's parent
  float z[16];
  float A = 0.f, zmax = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int ti = 8 * (j >> 2) + 4 * h + (j & 3);
    if (vt[ti] >= 0) {
      z[j] = lval[ti] + acc[j];
      A = fmaxf(A, aacc[j]);
      zmax = fmaxf(zmax, fabsf(z[j]));
    } else {
      z[j] = neg_inf();
    }
  }
  // k-th largest of the column's 32 values (16 here, 16 in lane^32)
  uint32_t removed = 0;
  float kth = neg_inf();
  for (int r = 0; r < sa.k; ++r) {
    float bz = neg_inf();
    int bj = -1;
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (!((removed >> j) & 1u) && z[j] > bz) {
        bz = z[j];
        bj = j;
      }
    const float oz = swap_halves(bz, lane);
    const bool mine = bz > oz || (bz == oz && h == 0);
    if (mine && bj >= 0) removed |= 1u << bj;
    kth = fmaxf(bz, oz);
  }
  A = fmaxf(A, swap_halves(A, lane));
  zmax = fmaxf(zmax, swap_halves(zmax, lane));
  const float margin = 4.f * (float)sa.r * 5.9604645e-8f * A +
                       4.f * 1.1920929e-7f * zmax + 1e-30f;
  return kth - margin;
}

// Cooperative staging of the seed operands of L row `row`: the kSeedT seed
// tokens, their logits and W rows (all threads of the block take part).
__device__ void stage_seed_rows(const SeedArgs& sa, int row, uint4* wrows,
                                float* lval, int* vt, int tid, int nthr) {
  const int* rt = sa.rowtop + (int64_t)row * kSeedT;
  const int ch = sa.r / 8, cs = ch + 1;
  for (int i = tid; i < kSeedT * ch; i += nthr) {
    const int t = i / ch, c = i % ch;
    const int v = rt[t];
    const int vv = (v >= 0 && v < sa.V) ? v : 0;
    wrows[t * cs + c] =
        reinterpret_cast<const uint4*>(sa.W)[(int64_t)vv * ch + c];
  }
  for (int t = tid; t < kSeedT; t += nthr) {
    const int v = rt[t];
    const bool ok = v >= 0 && v < sa.V;
    vt[t] = ok ? v : -1;
    lval[t] = ok ? sa.L[(int64_t)row * sa.lstride + v] : 0.f;
  }
}

// Cooperative staging of the U rows of up to 32 parents.
__device__ void stage_parent_rows(const SeedArgs& sa, const int32_t* ptok,
                                  int npar, uint4* urows, int tid, int nthr) {
  const int ch = sa.r / 8, cs = ch + 1;
  for (int i = tid; i < 32 * ch; i += nthr) {
    const int t = i / ch, c = i % ch;
    const int tok = t < npar ? min(max(ptok[t], 0), sa.V - 1) : 0;
    urows[t * cs + c] =
        reinterpret_cast<const uint4*>(sa.U)[(int64_t)tok * ch + c];
  }
}

constexpr int kSeedRowChunks = 256 / 8 + 1;  // r <= 256, one pad chunk

__device__ __forceinline__ bool seed_by_mfma(const SeedArgs& sa) {
  return sa.use_seed && sa.U != nullptr && sa.uw_bf16 && sa.r % 16 == 0 &&
         sa.r <= 256 && sa.k <= kSeedT;
}

__device__ float seed_theta_mfma_split(const SeedArgs& sa, const uint4* wrows,
                                       const int32_t* ptok, int npar,
                                       const float* lval, const int* vt,
                                       float* red, int tid,
                                       uint4* upack = nullptr, int pbase = 0);

// ---------------------------------------------------------------------
// Depth-1 frontier: the anchor of each request.
// Four waves stage the seed operands (their loads in flight together); the
// first wave computes the threshold.
constexpr int kInitThreads = 256;
__global__ __launch_bounds__(kInitThreads) void init_kernel(
    int B, const int32_t* anchor, Frontier f, int32_t* gcnt, int32_t* tq,
    int n_tq, SeedArgs sa) {
  static_assert(kInitThreads == 256, "four waves (the split seed routine)");
  __shared__ uint4 wrows[kSeedT * kSeedRowChunks];
  __shared__ float red[3 * 32 * 64];
  __shared__ float lval[kSeedT];
  __shared__ int vt[kSeedT];
  const int q = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  const int a = anchor[q];
  const bool mf = seed_by_mfma(sa);
  float th = 0.f;
  if (mf) {
    // the seed tokens of row q*B, then their W rows (four 16-byte chunks
    // per thread, every load issued before any store)
    const int ch = sa.r / 8, cs = ch + 1;
    const int* rt = sa.rowtop + (int64_t)q * B * kSeedT;
    int wtok[4];
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int i = tid + it * kInitThreads;
      wtok[it] = i < kSeedT * ch ? rt[i / ch] : -1;
    }
    uint4 wpre[4];
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int i = tid + it * kInitThreads;
      const int v = wtok[it];
      const int vv = (v >= 0 && v < sa.V) ? v : 0;
      wpre[it] = make_uint4(0, 0, 0, 0);
      if (i < kSeedT * ch)
        wpre[it] =
            reinterpret_cast<const uint4*>(sa.W)[(int64_t)vv * ch + i % ch];
    }
    if (tid < kSeedT) {
      const int v = rt[tid];
      const bool ok = v >= 0 && v < sa.V;
      vt[tid] = ok ? v : -1;
      lval[tid] = ok ? sa.L[(int64_t)q * B * sa.lstride + v] : 0.f;
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int i = tid + it * kInitThreads;
      if (i < kSeedT * ch) wrows[(i / ch) * cs + i % ch] = wpre[it];
    }
    __syncthreads();
    // with the packed U row of this parent (parent q of the depth-1
    // frontier), which the MFMA block loads anyway
    th = seed_theta_mfma_split(sa, wrows, anchor + q, 1, lval, vt, red, tid,
                               sa.upack, q);
  }
  if (!mf && sa.upack != nullptr) {
    // packed U row of this parent (parent q of the depth-1 frontier)
    const int ch = sa.r / 8;
    const uint4* urow = reinterpret_cast<const uint4*>(sa.U) +
                        (int64_t)min(max(a, 0), sa.V - 1) * ch;
    for (int c = tid; c < ch; c += kInitThreads)
      sa.upack[upack_index(q, c, ch / 2)] = urow[c];
  }
  // the fused kernel's tile queue starts the build cleared (every launch
  // leaves it cleared)
  if (q == 0)
    for (int i = tid; i < n_tq; i += kInitThreads) tq[i] = 0;
  if (tid >= 64) return;
  if (!mf) th = seed_theta(sa, a, q * B, lane);
  if (lane == 0) {
    f.tok[q] = a;
    f.pid[q] = -1;
    f.lrow[q] = q * B;
    f.s[q] = 0.f;
    f.theta[q] = th;
    gcnt[q] = 0;
  }
}

// The log-normaliser of one parent from its (c, s) partials, one wave:
// part(i) returns partial i of S.  Each lane keeps a running (max, sum) with
// a double sum; lanes combine by DPP reductions.
template <typename F>
__device__ float wave_lse_from(F&& part, int S, int lane) {
  float cm = neg_inf();
  double acc = 0.0;
  for (int i = lane; i < S; i += kWave) {
    const float2 cv = part(i);
    if (cv.x == neg_inf() || !(cv.y > 0.f)) continue;
    if (cv.x > cm) {
      acc = acc * (double)__builtin_amdgcn_exp2f(cm - cv.x) + (double)cv.y;
      cm = cv.x;
    } else {
      acc += (double)cv.y * (double)__builtin_amdgcn_exp2f(cv.x - cm);
    }
  }
  const float gm = wave_max(cm);
  acc = (cm == neg_inf()) ? 0.0
                          : acc * (double)__builtin_amdgcn_exp2f(cm - gm);
  acc = wave_sum(acc);
  return (float)(kLn2 * ((double)gm + log2(acc)));
}

// One workgroup per request: children of every frontier parent, their
// scores and pool keys, the beam of the next depth and its seeds.
//  1. all independent loads first: the next row's seed tokens, their logits
//     and W rows; the partials of up to 8 parents, read coalesced ([S][P]
//     rows of consecutive parents) into LDS;
//  2. one wave per parent: log-normaliser and top-k of its candidates;
//  3. the beam (rank of each child's key);
//  4. the new parents' seed thresholds for the next depth as one MFMA block
//     per 32 of them (their U rows pass through its operand registers into
//     the packed rows of the next depth), or one wave per new parent when
//     the seeds cannot use MFMA.
// Eight waves: the MFMA seed block needs more than the 128 registers a
// 1024-thread workgroup allows; the single kernel serves frontiers below 64
// parents in all (batch-1 builds, depth 1), at most 8 parents per request
// in the benchmark's workloads.
constexpr int kExpandWaves = 8;
constexpr int kStageSlices = 256;  // partials per parent staged in LDS
__global__ __launch_bounds__(kExpandWaves * 64) void expand_kernel(
    ExpandArgs a) {
  __shared__ uint64_t ckey[kMaxCand];
  __shared__ int32_t cpid[kMaxCand];
  __shared__ int32_t ctok[kMaxCand];
  __shared__ int32_t crank[kMaxCand];
  __shared__ float2 pst[kExpandWaves * kStageSlices];
  // child index of each beam rank (the partials are consumed by then)
  int32_t* bcand = reinterpret_cast<int32_t*>(pst);
  static_assert(sizeof(pst) >= (kMaxCand + kExpandWaves * kSeedT) * 4,
                "beam indices and seed scratch");
  __shared__ uint4 wrows[kSeedT * kSeedRowChunks];
  __shared__ float red[3 * 32 * 64];  // the seed block's partial sums
  __shared__ float lval[kSeedT];
  __shared__ int vt[kSeedT];
  constexpr int NT = kExpandWaves * 64;
  const int q = blockIdx.x, tid = threadIdx.x, lane = tid & 63,
            wave = tid >> 6;
  const int NC = a.Fp * a.k;
  const int row = q * a.B + a.d;  // L row of depth d+1
  const bool lseed = a.d < a.B && seed_by_mfma(a.seed);  // bf16, r <= 256
  const bool staged = !a.shared_stats && a.n_slices <= kStageSlices;
  // partials of a group of up to 8 parents into LDS; the first group's
  // loads are issued before the seed staging so that the two overlap
  constexpr int kStageIt = kExpandWaves * kStageSlices / NT;
  float2 pre[kStageIt];
  auto load_group = [&](int g0) {
    const int ng = min(kExpandWaves, a.Fp - g0);
    const int p0 = q * a.Fp + g0, S = a.n_slices;
#pragma unroll
    for (int it = 0; it < kStageIt; ++it) {
      const int e = tid + it * NT;
      pre[it] = make_float2(neg_inf(), 0.f);
      if (e < S * ng) {
        const int64_t o = (int64_t)(e / ng) * a.Pstat + p0 + e % ng;
        pre[it] = make_float2(a.part_c[o], a.part_s[o]);
      }
    }
  };
  auto store_group = [&](int g0) {
    const int ng = min(kExpandWaves, a.Fp - g0), S = a.n_slices;
#pragma unroll
    for (int it = 0; it < kStageIt; ++it) {
      const int e = tid + it * NT;
      if (e < S * ng) pst[(e % ng) * kStageSlices + e / ng] = pre[it];
    }
  };
  if (staged) load_group(0);
  // the first 64 candidate slots of this wave's first parent, loaded now so
  // that they arrive while the partials and the seed operands are staged
  // (slots past the parent's count are never used)
  float hz = neg_inf();
  int32_t hv = 0x7fffffff;
  if (wave < a.Fp && lane < a.cap) {
    const int64_t o =
        (int64_t)(a.shared_stats ? q : q * a.Fp + wave) * a.cap + lane;
    hz = a.gz[o];
    hv = a.gv[o];
  }
  if (lseed)
    stage_seed_rows(a.seed, row, wrows, lval, vt, tid, NT);
  for (int i = tid; i < NC; i += NT) crank[i] = 0;

  for (int g0 = 0; g0 < a.Fp; g0 += kExpandWaves) {
    const int ng = min(kExpandWaves, a.Fp - g0);
    if (staged) {
      if (g0 > 0) {
        __syncthreads();  // the previous group is consumed
        load_group(g0);
      }
      store_group(g0);
      __syncthreads();
    }
    const int j = g0 + wave;
    if (wave < ng) {
      const int p = q * a.Fp + j;
      const int sp = a.shared_stats ? q : p;
      const float sp_score = a.cur.s[p];
      const int ppid = a.cur.pid[p];
      const int cnt = min(a.gcnt[sp], a.cap);
      float lse;
      if (staged) {
        const float2* pp = pst + wave * kStageSlices;
        lse = wave_lse_from([&](int i) { return pp[i]; }, a.n_slices, lane);
      } else {
        lse = wave_lse_from(
            [&](int i) {
              const int64_t o = (int64_t)i * a.Pstat + sp;
              return make_float2(a.part_c[o], a.part_s[o]);
            },
            a.n_slices, lane);
      }
      // the wave's partials are consumed: its LDS rows serve as scratch
      wave_topk_rank(a.gz + (int64_t)sp * a.cap, a.gv + (int64_t)sp * a.cap,
                     cnt, a.k, lane, pst + wave * kStageSlices,
                     [&](int i, float z, int32_t v) {
                       // log pi(v|p); the merged lse can land an ulp below
                       // the row maximum on a near one-hot row, while the
                       // true value is never positive
                       const float l = fminf(z - lse, 0.f);
                       float s = sp_score + l;        // path score
                       s = s + 0.0f;                  // -0 -> +0
                       const int c = j * a.k + i;
                       const int pid = a.base_d + c;
                       const uint64_t key = make_key(s, ppid, v);
                       ckey[c] = key;
                       cpid[c] = pid;
                       ctok[c] = v;
                       a.pool_key[(int64_t)q * a.pool_n + pid] = key;
                     }, g0 == 0, hz, hv);
    }
  }
  __syncthreads();

  // beam: the Fn smallest keys of this depth's children (keys are distinct:
  // (parent, token) pairs are unique); rank counts split over the threads
  const int parts = NC <= NT ? max(1, NT / NC) : 1;
  if (NC <= NT) {
    const int c = tid % NC, part = tid / NC;
    if (part < parts) {
      const uint64_t key = ckey[c];
      const int o0 = (int)((int64_t)NC * part / parts);
      const int o1 = (int)((int64_t)NC * (part + 1) / parts);
      int r = 0;
      for (int o = o0; o < o1; ++o) r += ckey[o] < key;
      atomicAdd(&crank[c], r);
    }
  } else {
    for (int c = tid; c < NC; c += NT) {
      const uint64_t key = ckey[c];
      int r = 0;
      for (int o = 0; o < NC; ++o) r += ckey[o] < key;
      crank[c] = r;
    }
  }
  __syncthreads();
  for (int c = tid; c < NC; c += NT) {
    const int rank = crank[c];
    if (rank < a.Fn) {
      const uint64_t key = ckey[c];
      const int o = q * a.Fn + rank;
      a.nxt.tok[o] = key_tok(key);
      a.nxt.pid[o] = cpid[c];
      a.nxt.s[o] = key_score(key);
      a.nxt.lrow[o] = row;  // row of depth d+1
      bcand[rank] = c;
      if (a.gcnt_next) a.gcnt_next[o] = 0;
    }
  }
  if (a.d >= a.B) return;
  __syncthreads();

  if (lseed) {
    // the new parents' tokens in rank order (the ranks are consumed)
    int32_t* stok = crank;
    for (int i = tid; i < a.Fn; i += NT) stok[i] = ctok[bcand[i]];
    __syncthreads();
    for (int b0 = 0; b0 < a.Fn; b0 += 32) {
      const int nb = min(32, a.Fn - b0);
      const float th = seed_theta_mfma_split(a.seed, wrows, stok + b0, nb,
                                             lval, vt, red, tid, a.seed.upack,
                                             q * a.Fn + b0);
      if (tid < nb) a.nxt.theta[q * a.Fn + b0 + tid] = th;
      __syncthreads();  // red is rewritten by the next block
    }
    return;
  }
  // seeds without MFMA, one wave per new parent
  for (int i = wave; i < a.Fn; i += kExpandWaves) {
    const float th = seed_theta(a.seed, ctok[bcand[i]], row, lane);
    if (lane == 0) a.nxt.theta[q * a.Fn + i] = th;
  }
  // packed U rows of the next depth's parents (the fused kernel's operand
  // order)
  if (a.seed.upack != nullptr) {
    const uint4* Ug = reinterpret_cast<const uint4*>(a.seed.U);
    const int cr = a.seed.r / 8;
    for (int i = tid; i < a.Fn * cr; i += NT) {
      const int j = i / cr, c = i % cr;
      const int tok = min(max(ctok[bcand[j]], 0), a.seed.V - 1);
      a.seed.upack[upack_index(q * a.Fn + j, c, cr / 2)] =
          Ug[(int64_t)tok * cr + c];
    }
  }
}

// ---------------------------------------------------------------------
// The expand step split in two, for bf16 factors with seeds by MFMA:
//  merge_kernel  one wave per parent, ppw parents of one request per
//                workgroup (ppw * k <= 32): log-normaliser and top-k of the
//                parent's candidates, child scores and keys (the pool keys,
//                and the request's child keys for the beam).  The
//                per-parent work, which dominates the single-kernel form,
//                spreads over the chip instead of 16 waves per request on
//                one compute unit.
//  beam_kernel   one workgroup per request: the Fn best child keys become
//                the next frontier, with their seed thresholds for the next
//                depth (the survivors' U rows as the columns of one MFMA
//                block per 32 of them, against the next row's seed tokens,
//                staged while the keys are ranked) and packed U rows (not
//                launched at the last depth, whose frontier is unused).
constexpr int kMergeMaxWaves = 4;

// seed_theta_mfma spread over the four waves of a workgroup: wave w takes
// rank steps w, w+4, ... of the MFMA chain (its fragments all loaded before
// its MFMAs: the W rows of the seed tokens from LDS, staged by the caller;
// the U rows of up to 32 parents straight from global memory, their tokens
// in ptok), the partial sums meet in LDS (red: 3 x 2 x 16 x 64 floats),
// and wave 0 finishes as seed_theta_mfma does, with the same arithmetic
// and margin.  Every thread of the workgroup calls it (waves past the
// fourth only join its barrier); the result is meaningful in wave 0 only.
__device__ float seed_theta_mfma_split(const SeedArgs& sa, const uint4* wrows,
                                       const int32_t* ptok, int npar,
                                       const float* lval, const int* vt,
                                       float* red, int tid, uint4* upack,
                                       int pbase) {
  const int lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, col = lane & 31;
  const int ch = sa.r / 8, cs = ch + 1, steps = sa.r / 16;
  const int tok = col < npar ? min(max(ptok[col], 0), sa.V - 1) : 0;
  const uint4* ug = reinterpret_cast<const uint4*>(sa.U) + (int64_t)tok * ch;
  // waves 0-3 split the rank steps; any further waves of the workgroup only
  // take part in the barrier
  uint4 wf[4], uf[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int kk = wave + 4 * i;
    if (wave < 4 && kk < steps) {
      uf[i] = ug[2 * kk + h];
      wf[i] = wrows[col * cs + 2 * kk + h];
    }
  }
  f32x16 acc, aacc;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    acc[j] = 0.f;
    aacc[j] = 0.f;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (wave < 4 && wave + 4 * i < steps) {
      const uint4 w4 = wf[i], u4 = uf[i];
      const uint4 wa = make_uint4(w4.x & 0x7fff7fffu, w4.y & 0x7fff7fffu,
                                  w4.z & 0x7fff7fffu, w4.w & 0x7fff7fffu);
      const uint4 ua = make_uint4(u4.x & 0x7fff7fffu, u4.y & 0x7fff7fffu,
                                  u4.z & 0x7fff7fffu, u4.w & 0x7fff7fffu);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          __builtin_bit_cast(bf16x8, w4), __builtin_bit_cast(bf16x8, u4), acc,
          0, 0, 0);
      aacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          __builtin_bit_cast(bf16x8, wa), __builtin_bit_cast(bf16x8, ua), aacc,
          0, 0, 0);
    }
  }
  // the parents' U rows pass through these registers whole: written
  // packed in the fused kernel's operand order when asked for (parent
  // pbase + col)
  if (upack != nullptr && col < npar) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kk = wave + 4 * i;
      if (wave < 4 && kk < steps)
        upack[upack_index(pbase + col, 2 * kk + h, steps)] = uf[i];
    }
  }
  if (wave > 0 && wave < 4) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      red[((wave - 1) * 32 + j) * 64 + lane] = acc[j];
      red[((wave - 1) * 32 + 16 + j) * 64 + lane] = aacc[j];
    }
  }
  __syncthreads();
  if (wave > 0) return 0.f;
  // partial sums in rank-step order of the waves: the sum is the same
  // exact products as one chain, rounded in another order (the margin
  // bounds either)
#pragma unroll
  for (int w = 0; w < 3; ++w)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      acc[j] += red[(w * 32 + j) * 64 + lane];
      aacc[j] += red[(w * 32 + 16 + j) * 64 + lane];
    }
  // register j holds seed token 8*(j/4) + 4h + j%4 of this column's parent
  // (the token and logit reads all issued first, the test as a select)
  float z[16];
  int tv[16];
  float lv[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int ti = 8 * (j >> 2) + 4 * h + (j & 3);
    tv[j] = vt[ti];
    lv[j] = lval[ti];
  }
  float A = 0.f, zmax = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const bool ok = tv[j] >= 0;
    const float zj = lv[j] + acc[j];
    z[j] = ok ? zj : neg_inf();
    A = ok ? fmaxf(A, aacc[j]) : A;
    zmax = ok ? fmaxf(zmax, fabsf(zj)) : zmax;
  }
  // k-th largest of the column's 32 values (16 here, 16 in lane^32): each
  // half sorts its 16 values (descending, a bitonic network of max/min),
  // takes the other half's first k, and the k-th largest of the two sorted
  // lists a, b is max over i of min(a_i, b_{k-i}) (1-based, a_0 = b_0 =
  // +inf) -- the same value as k rounds of arg-max
#pragma unroll
  for (int s2 = 2; s2 <= 16; s2 <<= 1)
#pragma unroll
    for (int jj = s2 >> 1; jj > 0; jj >>= 1)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int l = i ^ jj;
        if (l > i) {
          const float x = z[i], y = z[l];
          // descending blocks where (i & s2) == 0, ascending otherwise; the
          // last merge (s2 = 16) is all descending
          if ((i & s2) == 0) {
            z[i] = fmaxf(x, y);
            z[l] = fminf(x, y);
          } else {
            z[i] = fminf(x, y);
            z[l] = fmaxf(x, y);
          }
        }
      }
  // the other half's sorted values through LDS (an index that depends on
  // k would otherwise index registers); red is free again once wave 0 has
  // read the partial sums
  float* srt = red + lane * 17;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int i = 0; i < 16; ++i) srt[i] = z[i];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const float* other = red + (lane ^ 32) * 17;
  const int k = sa.k;
  // every read issued before any is used (clamped in-range addresses), the
  // range test applied as a select
  float ob[17];
#pragma unroll
  for (int i = 0; i <= 16; ++i) ob[i] = other[min(max(k - i - 1, 0), 15)];
  float kth = neg_inf();
#pragma unroll
  for (int i = 0; i <= 16; ++i) {
    // i values from this half, k - i from the other
    const int jb = k - i;
    const float ai = i == 0 ? pos_inf() : z[i - 1];
    const float bj = jb == 0 ? pos_inf() : ob[i];
    const float m = fmaxf(kth, fminf(ai, bj));
    kth = (jb >= 0 && jb <= 16) ? m : kth;
  }
  A = fmaxf(A, swap_halves(A, lane));
  zmax = fmaxf(zmax, swap_halves(zmax, lane));
  const float margin = 4.f * (float)sa.r * 5.9604645e-8f * A +
                       4.f * 1.1920929e-7f * zmax + 1e-30f;
  return kth - margin;
}

bool expand_split_ok(const ExpandArgs& a) {
  const SeedArgs& s = a.seed;
  return !a.shared_stats && s.use_seed && s.U != nullptr && s.uw_bf16 &&
         s.r % 16 == 0 && s.r <= 256 && s.k <= kSeedT &&
         s.upack != nullptr && a.n_slices <= kStageSlices && a.ckey &&
         a.ppw >= 1 && a.ppw <= kMergeMaxWaves &&
         a.ppw * a.k <= 32 && a.Fp * a.k <= kMaxCand;
}

__global__ __launch_bounds__(kMergeMaxWaves * 64) void merge_kernel(
    ExpandArgs a) {
  __shared__ float2 pst[kMergeMaxWaves * kStageSlices];
  const int q = blockIdx.y, tid = threadIdx.x, lane = tid & 63,
            wave = tid >> 6;
  constexpr int NT = kMergeMaxWaves * 64;  // waves past the parents only stage
  const int j0 = blockIdx.x * a.ppw;
  const int npar = min(a.ppw, a.Fp - j0);
  const int S = a.n_slices;
  const int p0 = q * a.Fp + j0;
  const int NC = a.Fp * a.k;
  // 1. every load first: the partials of the workgroup's parents ([S][P]
  // rows of consecutive parents), the first 64 candidate slots and the
  // candidate count of this wave's parent
  // S * npar <= kStageSlices * ppw <= 4 * NT elements: at most 4 per thread
  constexpr int kIt = kStageSlices * kMergeMaxWaves / NT;
  const int total = S * npar;
  float2 pre[kIt];
#pragma unroll
  for (int it = 0; it < kIt; ++it) {
    const int e = tid + it * NT;
    pre[it] = make_float2(neg_inf(), 0.f);
    if (e < total) {
      const int64_t o = (int64_t)(e / npar) * a.Pstat + p0 + e % npar;
      pre[it] = make_float2(a.part_c[o], a.part_s[o]);
    }
  }
  const bool mine = wave < npar;
  const int j = j0 + wave;
  const int p = q * a.Fp + (mine ? j : j0);
  float hz = neg_inf();
  int32_t hv = 0x7fffffff;
  if (lane < a.cap) {
    hz = a.gz[(int64_t)p * a.cap + lane];
    hv = a.gv[(int64_t)p * a.cap + lane];
  }
  const int cnt = min(a.gcnt[p], a.cap);
  const float sp_score = a.cur.s[p];
  const int ppid = a.cur.pid[p];
#pragma unroll
  for (int it = 0; it < kIt; ++it) {
    const int e = tid + it * NT;
    if (e < total) pst[(e % npar) * kStageSlices + e / npar] = pre[it];
  }
  __syncthreads();

  // 2. one wave per parent: log-normaliser, top-k, child keys
  if (mine) {
    const float2* pp = pst + wave * kStageSlices;
    const float lse =
        wave_lse_from([&](int i) { return pp[i]; }, S, lane);
    // the wave's partials are consumed: its LDS rows serve as scratch
    wave_topk_rank(a.gz + (int64_t)p * a.cap, a.gv + (int64_t)p * a.cap, cnt,
                   a.k, lane, pst + wave * kStageSlices,
                   [&](int i, float z, int32_t v) {
                     // log pi(v|p), never positive (see expand_kernel)
                     const float l = fminf(z - lse, 0.f);
                     float s = sp_score + l;
                     s = s + 0.0f;
                     const int c = j * a.k + i;
                     const uint64_t key = make_key(s, ppid, v);
                     a.pool_key[(int64_t)q * a.pool_n + a.base_d + c] = key;
                     a.ckey[(int64_t)q * NC + c] = key;
                   },
                   true, hz, hv);
  }
}

constexpr int kBeamThreads = 512;  // the seed block needs > 128 registers
__global__ __launch_bounds__(kBeamThreads) void beam_kernel(ExpandArgs a) {
  __shared__ __align__(16) uint64_t ckey[kMaxCand];
  __shared__ int32_t crank[kMaxCand];
  __shared__ int32_t bcand[kMaxCand];
  // the next row's seed operands and the survivors' seed thresholds
  __shared__ uint4 wrows[kSeedT * kSeedRowChunks];
  __shared__ float red[3 * 32 * 64];
  __shared__ float lval[kSeedT];
  __shared__ int vt[kSeedT];
  __shared__ int32_t stok[32];
  constexpr int NT = kBeamThreads;
  const int q = blockIdx.x, tid = threadIdx.x;
  const int NC = a.Fp * a.k;
  const int row = q * a.B + a.d;  // L row of depth d+1
  // every independent load first: the next row's seed tokens, the child
  // keys, then the seed tokens' W rows (16-byte chunks, kWIt per thread)
  constexpr int kWIt = kSeedT * (kSeedRowChunks - 1) / NT;
  const int ch = a.seed.r / 8, cs = ch + 1;
  const int* rt = a.seed.rowtop + (int64_t)row * kSeedT;
  int wtok[kWIt];
#pragma unroll
  for (int it = 0; it < kWIt; ++it) {
    const int i = tid + it * NT;
    wtok[it] = i < kSeedT * ch ? rt[i / ch] : -1;
  }
  for (int c = tid; c < NC; c += NT) {
    ckey[c] = a.ckey[(int64_t)q * NC + c];
    crank[c] = 0;
  }
  uint4 wpre[kWIt];
#pragma unroll
  for (int it = 0; it < kWIt; ++it) {
    const int i = tid + it * NT;
    const int v = wtok[it];
    const int vv = (v >= 0 && v < a.seed.V) ? v : 0;
    wpre[it] = make_uint4(0, 0, 0, 0);
    if (i < kSeedT * ch)
      wpre[it] = reinterpret_cast<const uint4*>(a.seed.W)[(int64_t)vv * ch +
                                                          i % ch];
  }
  if (tid < kSeedT) {
    const int v = rt[tid];
    const bool ok = v >= 0 && v < a.seed.V;
    vt[tid] = ok ? v : -1;
    lval[tid] = ok ? a.seed.L[(int64_t)row * a.seed.lstride + v] : 0.f;
  }
#pragma unroll
  for (int it = 0; it < kWIt; ++it) {
    const int i = tid + it * NT;
    if (i < kSeedT * ch) wrows[(i / ch) * cs + i % ch] = wpre[it];
  }
  __syncthreads();
  // rank of every child key (keys are distinct: (parent, token) pairs are
  // unique); the counts are split over the threads
  if (NC <= NT) {
    const int parts = max(1, NT / NC);
    const int c = tid % NC, part = tid / NC;
    if (part < parts) {
      const uint64_t key = ckey[c];
      const int o0 = (int)((int64_t)NC * part / parts);
      const int o1 = (int)((int64_t)NC * (part + 1) / parts);
      int r = 0;
      int o = o0;
      // pairs of keys per 16-byte read, four reads in flight
      if ((o0 & 1) == 0) {
        const ulonglong2* k2 = reinterpret_cast<const ulonglong2*>(ckey);
        for (; o + 8 <= o1; o += 8) {
          ulonglong2 x[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) x[u] = k2[(o >> 1) + u];
#pragma unroll
          for (int u = 0; u < 4; ++u) r += (x[u].x < key) + (x[u].y < key);
        }
      }
      for (; o < o1; ++o) r += ckey[o] < key;
      atomicAdd(&crank[c], r);
    }
  } else {
    for (int c = tid; c < NC; c += NT) {
      const uint64_t key = ckey[c];
      int r = 0;
      for (int o = 0; o < NC; ++o) r += ckey[o] < key;
      crank[c] = r;
    }
  }
  __syncthreads();
  for (int c = tid; c < NC; c += NT) {
    const int rank = crank[c];
    if (rank < a.Fn) {
      const uint64_t key = ckey[c];
      const int o = q * a.Fn + rank;
      a.nxt.tok[o] = key_tok(key);
      a.nxt.pid[o] = a.base_d + c;
      a.nxt.s[o] = key_score(key);
      a.nxt.lrow[o] = row;
      if (a.gcnt_next) a.gcnt_next[o] = 0;
      bcand[rank] = c;
    }
  }
  __syncthreads();
  // the survivors' seed thresholds for the next depth, 32 at a time: their
  // U rows are the columns of one MFMA block against the seed tokens
  for (int b0 = 0; b0 < a.Fn; b0 += 32) {
    const int nb = min(32, a.Fn - b0);
    if (tid < nb) stok[tid] = key_tok(ckey[bcand[b0 + tid]]);
    __syncthreads();
    // with the packed U rows of the same parents, which the MFMA block
    // loads anyway (the fused kernel's operand order)
    const float th = seed_theta_mfma_split(a.seed, wrows, stok, nb, lval, vt,
                                           red, tid, a.seed.upack,
                                           q * a.Fn + b0);
    if (tid < nb) a.nxt.theta[q * a.Fn + b0 + tid] = th;
    __syncthreads();  // stok and red are rewritten by the next block
  }
}

hipError_t launch_merge(const ExpandArgs& a, hipStream_t s) {
  const int gx = (a.Fp + a.ppw - 1) / a.ppw;
  hipLaunchKernelGGL(merge_kernel, dim3(gx, a.batch),
                     dim3(kMergeMaxWaves * 64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_beam(const ExpandArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(beam_kernel, dim3(a.batch), dim3(kBeamThreads), 0, s, a);
  return hipGetLastError();
}

// Global top-N of every generated child of one request.  A key's output
// position is its rank among the request's keys in (key asc, pool id asc):
// the number of keys that come before it.  Keys are distinct except for
// padding children (score -inf, token 0, same parent), so the pool-id term
// is only counted for those.  Four lanes share a key, each counting over a
// quarter of the keys (16-byte LDS reads, two keys each), and add their
// counts with quad DPP; a kept key's parent index is the rank of the
// parent's key, counted in the same pass.  A request's keys are split over
// several workgroups (blockIdx.x), so the whole chip takes part.
constexpr int kTopNThreads = 256;

__device__ __forceinline__ int quad_sum(int x) {
  x += dpp_i<kDppXor1>(x);
  x += dpp_i<kDppXor2>(x);
  return x;
}

// Keys before ka (pool id ea) and before kb (pool id eb) among the 2*npairs
// keys of k2 (the tail is padded with ~0, above every key), in one pass so
// that every LDS read serves both counts; lane `sub` of the quad takes pairs
// sub, sub+4, ...  All four lanes of a quad call it with the same keys.
__device__ __forceinline__ void rank2_of(const ulonglong2* k2, int npairs,
                                         uint64_t ka, int ea, uint64_t kb,
                                         int eb, int sub, int& ra, int& rb) {
  int x = 0, y = 0;
  if (key_score(ka) != neg_inf() && key_score(kb) != neg_inf()) {
#pragma unroll 8
    for (int j = sub; j < npairs; j += 4) {
      const ulonglong2 v = k2[j];
      x += (v.x < ka) + (v.y < ka);
      y += (v.x < kb) + (v.y < kb);
    }
  } else {
#pragma unroll 4
    for (int j = sub; j < npairs; j += 4) {
      const ulonglong2 v = k2[j];
      x += (v.x < ka) + (v.y < ka) + (v.x == ka && 2 * j < ea) +
           (v.y == ka && 2 * j + 1 < ea);
      y += (v.x < kb) + (v.y < kb) + (v.x == kb && 2 * j < eb) +
           (v.y == kb && 2 * j + 1 < eb);
    }
  }
  ra = quad_sum(x);
  rb = quad_sum(y);
}

__global__ __launch_bounds__(kTopNThreads) void topn_kernel(TopNArgs a,
                                                            int splits) {
  extern __shared__ __align__(16) unsigned char smem[];
  uint64_t* key = reinterpret_cast<uint64_t*>(smem);
  const ulonglong2* k2 = reinterpret_cast<const ulonglong2*>(smem);
  const int q = blockIdx.y, sp = blockIdx.x, tid = threadIdx.x;
  const int pn = a.pool_n, npairs = (pn + 1) / 2;
  for (int i = tid; i < 2 * npairs; i += kTopNThreads)
    key[i] = i < pn ? a.pool_key[(int64_t)q * pn + i] : ~(uint64_t)0;
  __syncthreads();
  const int n = min(a.N, pn);
  const int per = (pn + splits - 1) / splits;
  const int e0 = sp * per, e1 = min(e0 + per, pn);
  const int grp = tid >> 2, sub = tid & 3;
  for (int b0 = e0; b0 < e1; b0 += kTopNThreads / 4) {
    const int e = b0 + grp;  // the same for the four lanes of a quad
    if (e >= e1) continue;
    const uint64_t k = key[e];
    // the key's rank and its parent's (the parent is the output row the
    // node points to), counted together
    const int pp = key_ppid(k);
    int r, pr;
    rank2_of(k2, npairs, k, e, pp < 0 ? k : key[pp], pp < 0 ? e : pp, sub, r,
             pr);
    if (r >= n) continue;
    if (pp < 0) pr = -1;
    if (sub == 0) {
      int d = 1;
      while (d < a.B && e >= a.base[d + 1]) ++d;
      const int64_t o = (int64_t)q * a.N + r;
      a.tok[o] = key_tok(k);
      a.parent[o] = pr;
      a.depth[o] = d;
      a.score[o] = key_score(k);
    }
  }
  if (sp == 0) {
    for (int i = n + tid; i < a.N; i += kTopNThreads) {
      const int64_t o = (int64_t)q * a.N + i;
      a.tok[o] = -1;
      a.parent[o] = -1;
      a.depth[o] = 0;
      a.score[o] = neg_inf();
    }
    if (tid == 0) a.n_nodes[q] = n;
  }
}

// Global top-N of one request in one workgroup: a threshold select, then a
// sort of the kept keys only.  The order is that of topn_kernel: (key asc,
// pool id asc).
// 1. The pool's keys go to LDS.
// 2. Unless the whole pool is kept, a radix select over the 80-bit
//    composite (key, pool id), one byte per pass from the top, finds where
//    the n-th smallest lies: a pass counts the candidates (elements whose
//    decided bytes equal the chosen ones) per value of the next byte, and a
//    scan of the 256 counts picks the byte where the n-th falls.  It stops
//    as soon as every candidate with the chosen byte is kept.
// 3. The n kept elements are compacted, in any order.
// 4. They are sorted: runs of 64 places by counting, then neighbouring runs
//    merged level by level.  In a merge an element's place is its offset in
//    its own run plus the number of the partner run's elements that come
//    before it, found by binary search.
// 5. Place = rank = output row.  A node's parent row is the place of the
//    parent's pool id: ancestors are always kept, since a child's key comes
//    after its parent's (its score is not larger, and on equal scores the
//    parent's own parent has the smaller pool id).
constexpr int kTopSelThreads = 1024;
constexpr int kTopRun = 64;  // 2^6, the first merge level
constexpr int kTopSelMaxLds = 160 * 1024;
// element tag: pool id in bits 0-13, depth in bits 14-20
constexpr uint32_t kTagId = 0x3fffu;

__device__ __forceinline__ bool comp_before(uint64_t ka, uint32_t ta,
                                            uint64_t kb, uint32_t tb) {
  return ka < kb || (ka == kb && (ta & kTagId) < (tb & kTagId));
}

// Top `nb` bytes of the composite (key, id) against the same bytes of the
// chosen prefix (kp, ip): -1 before, 0 equal, 1 after.
__device__ __forceinline__ int prefix_cmp(uint64_t key, uint32_t id, int nb,
                                          uint64_t kp, uint32_t ip) {
  if (nb == 0) return 0;
  if (nb <= 8) {
    const int sh = 64 - 8 * nb;
    const uint64_t a = key >> sh, b = kp >> sh;
    return a < b ? -1 : (a > b ? 1 : 0);
  }
  if (key != kp) return key < kp ? -1 : 1;
  const int sh = 16 - 8 * (nb - 8);
  const uint32_t a = id >> sh, b = ip >> sh;
  return a < b ? -1 : (a > b ? 1 : 0);
}

// byte `lv` (0 = top) of the composite (key, 16-bit id)
__device__ __forceinline__ int comp_byte(uint64_t key, uint32_t id, int lv) {
  return lv < 8 ? (int)((key >> (56 - 8 * lv)) & 255u)
                : (int)((id >> (8 * (9 - lv))) & 255u);
}

// Binary searches of two elements of one thread, interleaved: on return
// lo0 (lo1) is the first place of [lo0, lo0 + n0) ([lo1, lo1 + n1)) whose
// element does not come before (x0, t0) ((x1, t1)).  An exhausted search
// reads place `safe` and ignores it.
__device__ __forceinline__ void search2(const uint64_t* k, const uint32_t* t,
                                        int safe, int& lo0, int n0,
                                        uint64_t x0, uint32_t t0, int& lo1,
                                        int n1, uint64_t x1, uint32_t t1) {
  while (n0 > 0 || n1 > 0) {
    const int h0 = n0 >> 1, h1 = n1 >> 1;
    const int m0 = n0 > 0 ? lo0 + h0 : safe;
    const int m1 = n1 > 0 ? lo1 + h1 : safe;
    const bool b0 = comp_before(k[m0], t[m0], x0, t0);
    const bool b1 = comp_before(k[m1], t[m1], x1, t1);
    if (n0 > 0) {
      lo0 = b0 ? m0 + 1 : lo0;
      n0 = b0 ? n0 - h0 - 1 : h0;
    }
    if (n1 > 0) {
      lo1 = b1 ? m1 + 1 : lo1;
      n1 = b1 ? n1 - h1 - 1 : h1;
    }
  }
}

__device__ __forceinline__ int sel_wave_scan(int x) {  // inclusive, 64 lanes
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // bcast:31
  return x;
}

// hist[d] += 1 for every lane with d >= 0.  The two values held by the
// most lanes (in early radix passes most lanes hold one of a few) are
// added once per wave; the rest with one atomic per lane.
__device__ __forceinline__ void hist_add(int* hist, int d, int lane) {
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const uint64_t act = __ballot(d >= 0);
    if (act == 0) return;
    const int f = __builtin_ctzll(act);
    const int v = __builtin_amdgcn_readlane(d, f);
    const uint64_t m = __ballot(d == v);
    if (lane == f) atomicAdd(&hist[v], __popcll(m));
    if (d == v) d = -1;
  }
  if (d >= 0) atomicAdd(&hist[d], 1);
}

__global__ __launch_bounds__(kTopSelThreads) void topn_select_kernel(
    TopNArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int hist[2][256];  // alternate passes
  __shared__ int sbase[66];
  __shared__ int sel[4];
  constexpr int T = kTopSelThreads;
  const int pn = a.pool_n, n = min(a.N, pn);
  const int ppad = (pn + 1) & ~1, npad = (n + 1) & ~1;
  uint64_t* pk = reinterpret_cast<uint64_t*>(smem);  // pool keys
  uint64_t* kc = pk + ppad;                          // kept, current order
  uint64_t* kn = kc + npad;                          // kept, next order
  uint32_t* tc = reinterpret_cast<uint32_t*>(kn + npad);
  uint32_t* tn = tc + npad;
  const int q = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  for (int p = tid; p < pn; p += T) pk[p] = a.pool_key[(int64_t)q * pn + p];
  if (tid <= a.B + 1) sbase[tid] = a.base[tid];
  if (tid == 0) sel[3] = 0;
  for (int i = tid; i < 512; i += T) (&hist[0][0])[i] = 0;
  __syncthreads();

  // 2. threshold: the chosen bytes (kp, ip) and how many of the bytes are
  // decided (nb); an element is kept when its top nb bytes are not after
  // the chosen ones
  uint64_t kp = 0;
  uint32_t ip = 0;
  int nb = 0;
  if (n < pn) {
    int need = n;
    for (int lv = 0; lv < 10; ++lv) {
      int* h = hist[lv & 1];
      // the other buffer was last read before the previous pass's second
      // barrier: clear it for the next pass
      for (int i = tid; i < 256; i += T) hist[(lv + 1) & 1][i] = 0;
      for (int p0 = 0; p0 < pn; p0 += T) {
        const int p = min(p0 + tid, pn - 1);
        const uint64_t x = pk[p];
        const bool cand = p0 + tid < pn &&
                          prefix_cmp(x, (uint32_t)p, lv, kp, ip) == 0;
        hist_add(h, cand ? comp_byte(x, (uint32_t)p, lv) : -1, lane);
      }
      __syncthreads();
      if (tid < 64) {
        const int h0 = h[4 * lane], h1 = h[4 * lane + 1],
                  h2 = h[4 * lane + 2], h3 = h[4 * lane + 3];
        const int incl = sel_wave_scan(h0 + h1 + h2 + h3);
        int ex = incl - (h0 + h1 + h2 + h3);
        if (ex < need && need <= incl) {
          int j = 0, hj = h0;
          if (need > ex + hj) { ex += hj; j = 1; hj = h1; }
          if (need > ex + hj) { ex += hj; j = 2; hj = h2; }
          if (need > ex + hj) { ex += hj; j = 3; hj = h3; }
          sel[0] = 4 * lane + j;
          sel[1] = ex;
          sel[2] = hj;
        }
      }
      __syncthreads();
      const int b = sel[0], before = sel[1], hb = sel[2];
      if (lv < 8)
        kp |= (uint64_t)b << (56 - 8 * lv);
      else
        ip |= (uint32_t)b << (8 * (9 - lv));
      need -= before;
      nb = lv + 1;
      if (hb == need) break;
    }
  }

  // 3. compaction of the n kept elements, with their tags
  for (int p0 = 0; p0 < pn; p0 += T) {
    const int p = p0 + tid;
    const bool keep =
        p < pn && (nb == 0 || prefix_cmp(pk[min(p, pn - 1)], (uint32_t)p, nb,
                                         kp, ip) <= 0);
    const uint64_t m = __ballot(keep);
    int w0 = 0;
    if (lane == 0 && m) w0 = atomicAdd(&sel[3], __popcll(m));
    w0 = __shfl(w0, 0);
    if (keep) {
      const int pos = w0 + __builtin_amdgcn_mbcnt_hi(
                               (uint32_t)(m >> 32),
                               __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
      int d = 1;
      while (d < a.B && p >= sbase[d + 1]) ++d;
      kn[pos] = pk[p];
      tn[pos] = (uint32_t)p | ((uint32_t)d << 14);
    }
  }
  __syncthreads();

  // 4a. runs of kTopRun places sorted by counting; four lanes per element
  // (a quad), each counting a quarter of the run
  for (int e0 = 0; e0 < n; e0 += T / 4) {
    const int e = min(e0 + (tid >> 2), n - 1), sub = tid & 3;
    const uint64_t x = kn[e];
    const uint32_t tx = tn[e];
    const int c0 = e & ~(kTopRun - 1), c1 = min(c0 + kTopRun, n);
    int r = 0;
#pragma unroll 4
    for (int j = c0 + sub; j < c1; j += 4)
      r += comp_before(kn[j], tn[j], x, tx);
    r = quad_sum(r);
    if (sub == 0 && e0 + (tid >> 2) < n) {
      kc[c0 + r] = x;
      tc[c0 + r] = tx;
    }
  }
  __syncthreads();
  const int runs = (n + kTopRun - 1) / kTopRun;
  if (runs > 1 && runs <= 8) {
    // 4b'. rank = offset in the own run + the elements of every other run
    // that come before it; lane `sub` of a quad searches runs sub, sub + 4
    for (int e0 = 0; e0 < n; e0 += T / 4) {
      const int e = min(e0 + (tid >> 2), n - 1), sub = tid & 3;
      const uint64_t x = kc[e];
      const uint32_t tx = tc[e];
      const int own = e / kTopRun;
      const int ra = sub, rb = sub + 4;
      int lo0 = ra * kTopRun, lo1 = rb * kTopRun;
      const int n0 = (ra < runs && ra != own) ? min(kTopRun, n - lo0) : 0;
      const int n1 = (rb < runs && rb != own) ? min(kTopRun, n - lo1) : 0;
      const int s0 = lo0, s1 = lo1;
      search2(kc, tc, e, lo0, n0, x, tx, lo1, n1, x, tx);
      int r = (lo0 - s0) + (lo1 - s1) + (sub == 0 ? e - own * kTopRun : 0);
      r = quad_sum(r);
      if (sub == 0 && e0 + (tid >> 2) < n) {
        kn[r] = x;
        tn[r] = tx;
      }
    }
    __syncthreads();
    uint64_t* kk = kc;
    kc = kn;
    kn = kk;
    uint32_t* tt = tc;
    tc = tn;
    tn = tt;
  }
  // 4b. otherwise merges; a run at this level is R = 2^lr places
  for (int lr = 6; runs > 8 && (1 << lr) < n; ++lr) {
    const int R = 1 << lr;
    for (int p0 = tid; p0 < n; p0 += 2 * T) {
      const int p1 = min(p0 + T, n - 1);  // a repeat of p0's work if past
      const uint64_t x0 = kc[p0], x1 = kc[p1];
      const uint32_t t0 = tc[p0], t1 = tc[p1];
      const int m0 = p0 >> lr, m1 = p1 >> lr;
      const int o0 = m0 ^ 1, o1 = m1 ^ 1;
      int lo0 = o0 * R, lo1 = o1 * R;
      const int n0 = max(0, min(lo0 + R, n) - lo0);
      const int n1 = max(0, min(lo1 + R, n) - lo1);
      const int s0 = lo0, s1 = lo1;
      search2(kc, tc, p0, lo0, n0, x0, t0, lo1, n1, x1, t1);
      const int np0 = n0 > 0 ? min(m0, o0) * R + (p0 - m0 * R) + (lo0 - s0)
                             : p0;
      const int np1 = n1 > 0 ? min(m1, o1) * R + (p1 - m1 * R) + (lo1 - s1)
                             : p1;
      kn[np0] = x0;
      tn[np0] = t0;
      if (p0 + T < n) {
        kn[np1] = x1;
        tn[np1] = t1;
      }
    }
    __syncthreads();
    uint64_t* kk = kc;
    kc = kn;
    kn = kk;
    uint32_t* tt = tc;
    tc = tn;
    tn = tt;
  }

  // 5. rows; the place of every kept pool id, in the pool-key array (free)
  int* rk = reinterpret_cast<int*>(pk);
  for (int r = tid; r < n; r += T) rk[tc[r] & kTagId] = r;
  __syncthreads();
  for (int r = tid; r < a.N; r += T) {
    const int64_t o = (int64_t)q * a.N + r;
    if (r < n) {
      const uint64_t x = kc[r];
      const int pp = key_ppid(x);
      a.tok[o] = key_tok(x);
      a.parent[o] = pp < 0 ? -1 : rk[pp];
      a.depth[o] = (int)((tc[r] >> 14) & 127u);
      a.score[o] = key_score(x);
    } else {
      a.tok[o] = -1;
      a.parent[o] = -1;
      a.depth[o] = 0;
      a.score[o] = neg_inf();
    }
  }
  if (tid == 0) a.n_nodes[q] = n;
}

// Per-parent results of the standalone Markov-logit call.
__global__ __launch_bounds__(256) void finalize_kernel(
    int P, int k, int S, const float* part_c, const float* part_s,
    const int32_t* gcnt, const float* gz, const int32_t* gv, int cap,
    float* lse_out, int32_t* topk_tok, float* topk_logp) {
  const int lane = threadIdx.x & 63;
  const int p = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (p >= P) return;
  float lse = wave_merge_lse(part_c, part_s, S, P, p, lane);
  const int cnt = min(gcnt[p], cap);
  wave_topk(gz + (int64_t)p * cap, gv + (int64_t)p * cap, cnt, k, lane,
            [&](int i, float z, int32_t v) {
              // the first result is the row maximum, a lower bound of the
              // true log-normaliser (every lane sees the same values)
              if (i == 0) lse = fmaxf(lse, z);
              if (lane == 0) {
                topk_tok[(int64_t)p * k + i] = v;
                topk_logp[(int64_t)p * k + i] = z - lse;
              }
            });
  if (lane == 0) lse_out[p] = lse;
}

// ---------------------------------------------------------------------

hipError_t launch_rowtop(const float* L, int rows, int V, int64_t lstride,
                         int vec_ok, int32_t* rowtop, hipStream_t s) {
  hipLaunchKernelGGL(row_top_kernel, dim3(rows, kRowTopPieces), dim3(256), 0,
                     s, L, V, lstride, vec_ok, rowtop);
  return hipGetLastError();
}

hipError_t launch_init(int batch, int B, const int32_t* anchor, Frontier f,
                       int32_t* gcnt, int32_t* tq, int n_tq,
                       const SeedArgs& sa, hipStream_t s) {
  hipLaunchKernelGGL(init_kernel, dim3(batch), dim3(kInitThreads), 0, s, B,
                     anchor, f, gcnt, tq, n_tq, sa);
  return hipGetLastError();
}

hipError_t launch_expand(const ExpandArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(expand_kernel, dim3(a.batch), dim3(kExpandWaves * 64), 0,
                     s, a);
  return hipGetLastError();
}

size_t topn_lds(int pool_n) { return (size_t)((pool_n + 1) / 2) * 16; }

static size_t topn_select_lds(int pool_n, int N) {
  const size_t pp = (size_t)((pool_n + 1) & ~1);
  const size_t n = (size_t)((std::min(N, pool_n) + 1) & ~1);
  return 8 * pp + 24 * n;
}

hipError_t launch_topn(const TopNArgs& a, hipStream_t s) {
  const size_t sl = topn_select_lds(a.pool_n, a.N);
  if (a.pool_n > 0 && a.N > 0 && sl + 2048 <= kTopSelMaxLds) {
    hipError_t e =
        allow_lds(reinterpret_cast<const void*>(topn_select_kernel), sl);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topn_select_kernel, dim3(a.batch), dim3(kTopSelThreads),
                       sl, s, a);
    return hipGetLastError();
  }
  hipError_t e = allow_lds(reinterpret_cast<const void*>(topn_kernel),
                           topn_lds(a.pool_n));
  if (e != hipSuccess) return e;
  // about 1024 workgroups over the batch, at least 64 keys each
  int splits = (1024 + a.batch - 1) / a.batch;
  splits = std::min(splits, std::max(1, (a.pool_n + 63) / 64));
  hipLaunchKernelGGL(topn_kernel, dim3(splits, a.batch), dim3(kTopNThreads),
                     topn_lds(a.pool_n), s, a, splits);
  return hipGetLastError();
}

hipError_t launch_finalize(int P, int k, int n_slices, const float* part_c,
                           const float* part_s, const int32_t* gcnt,
                           const float* gz, const int32_t* gv, int cap,
                           float* lse, int32_t* topk_tok, float* topk_logp,
                           hipStream_t s) {
  hipLaunchKernelGGL(finalize_kernel, dim3((P + 3) / 4), dim3(256), 0, s, P,
                     k, n_slices, part_c, part_s, gcnt, gz, gv, cap, lse,
                     topk_tok, topk_logp);
  return hipGetLastError();
}

}  // namespace pct
