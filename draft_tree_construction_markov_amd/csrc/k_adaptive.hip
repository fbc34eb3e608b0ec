// k_adaptive.hip -- the adaptive best-first draft tree over a block-diffusion
// drafter's per-position marginals (CaDDTree summary, "Method": for a fixed
// node count the best tree takes prefixes in order of probability; nodes are
// added one at a time and the build stops as soon as the throughput
// (1 + Phi) / (C_d + C_v(n; l)) no longer increases).
//
// Kernels:
//  rowpart_kernel / rowmerge_kernel  single-read row statistics: each logit
//                   row is read once, in register-resident pieces whose
//                   maxima, exp-sums and best K are merged per row.
//  rowsel_kernel    one workgroup per logit row: streaming log-sum-exp and
//                   the row's best K tokens (logit desc, token asc), exact:
//                   a pass computes per-thread bests, the K-th best of those
//                   bounds the row's K-th best from below, a second pass
//                   collects every element not after that bound, ranks them.
//  bestfirst_batched_kernel  one workgroup per request: the first K <= 64
//                   nodes of the best-first order by a threshold select
//                   (every prefix above a provable bound, then a radix
//                   select and exact ranking), and the stop test at every n
//                   at once.  Requests it cannot finish are flagged.
//  bestfirst_kernel one wave per request: lazy best-first expansion (a popped
//                   node pushes its next sibling and its first child) over
//                   the per-depth lists, with the stop test evaluated before
//                   every pop; it builds the flagged requests (from
//                   full-length lists when the short ones were outgrown).
#include <algorithm>

#include "pct_device.h"
#include "pct_internal.h"

namespace pct {

constexpr int kRowThreads = 1024;
constexpr int kRowCap = 4096;       // LDS candidate buffer of rowsel
constexpr int kFrontierCap = 4096;  // LDS frontier of bestfirst
constexpr int kPartThreads = 512;  // single-read row statistics
constexpr int kPartVec = 19;       // 16-byte loads per thread
constexpr int kPartCap = 2048;     // LDS candidate buffer of rowpart

struct RowSelArgs {
  const float* L;
  int V, B, K, kstride;
  const int32_t* only_flagged;  // null: every row; else rows of flagged reqs
  int vec_ok;
  float* lse;     // [rows]
  int32_t* ltok;  // [rows][kstride]
  float* llp;     // [rows][kstride]  log pi = fp32(L - lse)
};

// Single-read row statistics (see rowpart_kernel).
struct RowPartArgs {
  const float* L;
  int V, K, parts, chunk4;  // chunk4: 16-byte vectors per piece
  float* pm;    // [rows][parts] piece maximum, log2 units
  double* ps;   // [rows][parts] piece sum of 2^(z log2e - pm)
  float* cz;    // [rows][parts][K] piece best K, sorted; padding (-inf,
  int32_t* cv;  //   INT32_MAX)
};
struct RowMergeArgs {
  int K, parts, kstride;
  const float* pm;
  const double* ps;
  const float* cz;
  const int32_t* cv;
  float* lse;
  int32_t* ltok;
  float* llp;
};

__device__ __forceinline__ bool not_after(float z, int v, float tz, int tv) {
  return zv_before(z, v, tz, tv) || (z == tz && v == tv);
}

__global__ __launch_bounds__(kRowThreads) void rowsel_kernel(RowSelArgs a) {
  __shared__ float tbz[kRowThreads];
  __shared__ int tbv[kRowThreads];
  __shared__ float cz[kRowCap];
  __shared__ int cv[kRowCap];
  __shared__ float wm[kRowThreads / kWave];
  __shared__ float wz[kRowThreads / kWave];
  __shared__ double ws[kRowThreads / kWave];
  __shared__ int s_count;
  __shared__ float s_tz;
  __shared__ int s_tv;
  __shared__ float s_lse;
  const int row = blockIdx.x;
  if (a.only_flagged && !a.only_flagged[row / a.B]) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* Lr = a.L + (int64_t)row * a.V;

  // pass 1: online log-sum-exp (log2 units) and the thread's best element
  float m2 = neg_inf(), S = 0.f, bz = neg_inf();
  int bv = 0x7fffffff;
  auto visit = [&](float z, int v) {
    const float z2 = z * kLog2e;
    if (z2 > m2) {
      S = S * __builtin_amdgcn_exp2f(m2 - z2) + 1.f;
      m2 = z2;
    } else {
      S += __builtin_amdgcn_exp2f(z2 - m2);
    }
    if (zv_before(z, v, bz, bv)) {
      bz = z;
      bv = v;
    }
  };
  const int n4 = a.vec_ok ? a.V / 4 : 0;
  const float4* L4 = reinterpret_cast<const float4*>(Lr);
  for (int i0 = tid; i0 < n4; i0 += 4 * kRowThreads) {
    float4 x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + u * kRowThreads;
      x[u] = i < n4 ? L4[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + u * kRowThreads;
      if (i < n4) {
        visit(x[u].x, 4 * i);
        visit(x[u].y, 4 * i + 1);
        visit(x[u].z, 4 * i + 2);
        visit(x[u].w, 4 * i + 3);
      }
    }
  }
  for (int v = 4 * n4 + tid; v < a.V; v += kRowThreads) visit(Lr[v], v);

  // block log-sum-exp: lanes -> waves -> block, combined in double
  {
    const float wmax = wave_max(m2);
    const float sc = (m2 == neg_inf()) ? 0.f
                                       : S * __builtin_amdgcn_exp2f(m2 - wmax);
    const double wsum = wave_sum((double)sc);
    const float wbest = wave_max(bz);
    if (lane == 0) {
      wm[wave] = wmax;
      wz[wave] = wbest;
      ws[wave] = wsum;
    }
  }
  tbz[tid] = bz;
  tbv[tid] = bv;
  if (tid == 0) {
    s_count = 0;
    s_tz = neg_inf();  // "take everything" unless a K-th best exists
    s_tv = 0x7fffffff;
  }
  __syncthreads();
  if (tid == 0) {
    float M = wm[0];
    for (int w = 1; w < kRowThreads / kWave; ++w) M = fmaxf(M, wm[w]);
    double tot = 0.0;
    float zt = neg_inf();
    for (int w = 0; w < kRowThreads / kWave; ++w) {
      if (wm[w] != neg_inf()) tot += ws[w] * exp2((double)wm[w] - M);
      zt = fmaxf(zt, wz[w]);
    }
    // never below the row maximum (see rowmerge_kernel)
    s_lse = fmaxf((float)(kLn2 * ((double)M + log2(tot))), zt);
  }

  // bound: the K-th best of the group bests (K <= 256: groups of 4 threads)
  // or of the thread bests; K distinct elements are not after it, so it
  // cannot be after the row's K-th best
  if (a.K <= 256) {
    float gz = neg_inf();
    int gv = 0x7fffffff;
    if (tid < 256) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (zv_before(tbz[4 * tid + i], tbv[4 * tid + i], gz, gv)) {
          gz = tbz[4 * tid + i];
          gv = tbv[4 * tid + i];
        }
    }
    __syncthreads();
    if (tid < 256) {
      tbz[tid] = gz;
      tbv[tid] = gv;
    }
    __syncthreads();
    if (tid < 256) {
      int rank = 0;
      for (int j = 0; j < 256; ++j) rank += zv_before(tbz[j], tbv[j], gz, gv);
      if (rank == a.K - 1) {
        s_tz = gz;
        s_tv = gv;
      }
    }
  } else {
    int rank = 0;
    for (int j = 0; j < kRowThreads; ++j)
      rank += zv_before(tbz[j], tbv[j], bz, bv);
    if (rank == a.K - 1) {
      s_tz = bz;
      s_tv = bv;
    }
  }
  __syncthreads();
  float tz = s_tz;
  int tv = s_tv;
  if (tv == 0x7fffffff) tz = neg_inf();  // fewer than K elements: take all

  // pass 2 (repeated while the buffer overflows): collect every element not
  // after the bound
  for (;;) {
    if (tid == 0) s_count = 0;
    __syncthreads();
    auto offer = [&](float z, int v, bool valid) {
      const bool take = valid && not_after(z, v, tz, tv);
      const uint64_t bal = __ballot(take);
      if (bal == 0) return;
      int base = 0;
      if (lane == 0) base = atomicAdd(&s_count, __popcll(bal));
      base = __builtin_amdgcn_readfirstlane(base);
      if (take) {
        const int pos =
            base + __builtin_amdgcn_mbcnt_hi(
                       (uint32_t)(bal >> 32),
                       __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
        if (pos < kRowCap) {
          cz[pos] = z;
          cv[pos] = v;
        }
      }
    };
    for (int i0 = wave * kWave; i0 < n4; i0 += kRowThreads) {
      const int i = i0 + lane;
      const bool ok = i < n4;
      const float4 x = ok ? L4[i] : make_float4(0.f, 0.f, 0.f, 0.f);
      offer(x.x, 4 * i, ok);
      offer(x.y, 4 * i + 1, ok);
      offer(x.z, 4 * i + 2, ok);
      offer(x.w, 4 * i + 3, ok);
    }
    for (int v0 = 4 * n4 + wave * kWave; v0 < a.V; v0 += kRowThreads) {
      const int v = v0 + lane;
      offer(v < a.V ? Lr[v] : 0.f, v, v < a.V);
    }
    __syncthreads();
    const int count = s_count;
    if (count <= kRowCap) break;
    // overflow: the K-th best of the kRowCap collected elements is a
    // tighter bound; at least kRowCap - K elements drop out per round
    for (int e = tid; e < kRowCap; e += kRowThreads) {
      int rank = 0;
      for (int j = 0; j < kRowCap; ++j) rank += zv_before(cz[j], cv[j], cz[e], cv[e]);
      if (rank == a.K - 1) {
        s_tz = cz[e];
        s_tv = cv[e];
      }
    }
    __syncthreads();
    tz = s_tz;
    tv = s_tv;
  }
  const int count = s_count;
  const float lse = s_lse;
  // rank the collected elements; the first K form the list
  const int klist = min(a.K, count);
  for (int e = tid; e < count; e += kRowThreads) {
    const float z = cz[e];
    const int v = cv[e];
    int rank = 0;
    for (int j = 0; j < count; ++j) rank += zv_before(cz[j], cv[j], z, v);
    if (rank < klist) {
      a.ltok[(int64_t)row * a.kstride + rank] = v;
      a.llp[(int64_t)row * a.kstride + rank] = z - lse;  // log pi
    }
  }
  for (int r = klist + tid; r < a.K; r += kRowThreads) {
    a.ltok[(int64_t)row * a.kstride + r] = -1;
    a.llp[(int64_t)row * a.kstride + r] = neg_inf();
  }
  if (tid == 0) a.lse[row] = lse;
}

// ---------------------------------------------------------------------
// Single-read row statistics for short lists.  A row is cut into `parts`
// contiguous pieces; one workgroup per piece holds its piece in registers
// (at most kPartVec 16-byte loads per thread), so every logit is read from
// memory once.  A piece yields its maximum, its sum of exponentials relative
// to that maximum and its exact best K (logit desc, token asc), sorted.  The
// row's best K lie in the union of its pieces' best K, which the merge
// kernel ranks with one binary search per other piece.

__device__ __forceinline__ uint64_t zv_key(float z, int v) {
  // larger key = earlier in (logit desc, token asc)
  return ((uint64_t)float_to_ordered(z) << 32) | (uint32_t)(0x7fffffff - v);
}

__global__ __launch_bounds__(kPartThreads)
__attribute__((amdgpu_waves_per_eu(4))) void rowpart_kernel(RowPartArgs a) {
  __shared__ __align__(16) uint64_t ck[kPartCap + 8];
  __shared__ __align__(16) float gz[kPartThreads / 4];
  __shared__ float wmax[kPartThreads / kWave];
  __shared__ double wsum[kPartThreads / kWave];
  __shared__ int s_count;
  __shared__ float s_tz;
  __shared__ int s_tv;
  const int row = blockIdx.x, part = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n4 = a.V / 4;
  const int b4 = part * a.chunk4;
  const int e4 = min(b4 + a.chunk4, n4);  // > b4: pieces are never empty
  const float4* L4 =
      reinterpret_cast<const float4*>(a.L + (int64_t)row * a.V);

  // the piece, loaded once: unconditional loads (the tail repeats the last
  // in-range vector) so that every load is in flight before the first use;
  // non-temporal, since every logit is read once
  float4 x[kPartVec];
#pragma unroll
  for (int i = 0; i < kPartVec; ++i) {
    const f32x4 y = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(
        L4 + min(b4 + tid + i * kPartThreads, e4 - 1)));
    x[i] = make_float4(y.x, y.y, y.z, y.w);
  }
  // vectors i < nv of this thread are inside the piece; the rest become -inf
  const int nv = (e4 - b4 - tid + kPartThreads - 1) / kPartThreads;
#pragma unroll
  for (int i = 0; i < kPartVec; ++i) {
    const bool in = i < nv;
    x[i].x = in ? x[i].x : neg_inf();
    x[i].y = in ? x[i].y : neg_inf();
    x[i].z = in ? x[i].z : neg_inf();
    x[i].w = in ? x[i].w : neg_inf();
  }

  // thread maximum; the maxima of groups of 4 threads go to LDS
  float m = neg_inf();
#pragma unroll
  for (int i = 0; i < kPartVec; ++i)
    m = fmaxf(fmaxf(m, fmaxf(x[i].x, x[i].y)), fmaxf(x[i].z, x[i].w));
  float qm = fmaxf(m, Bits32<float>::from(dpp_i<kDppXor1>(Bits32<float>::to(m))));
  qm = fmaxf(qm, Bits32<float>::from(dpp_i<kDppXor2>(Bits32<float>::to(qm))));
  const float wm = wave_max(qm);
  if (lane == 0) wmax[wave] = wm;
  if ((lane & 3) == 0) gz[tid >> 2] = qm;
  if (tid == 0) {
    s_count = 0;
    s_tz = neg_inf();
  }
  __syncthreads();
  float M = wmax[0];
#pragma unroll
  for (int w = 1; w < kPartThreads / kWave; ++w) M = fmaxf(M, wmax[w]);
  const float M2 = M * kLog2e;

  // sum of 2^(z log2e - M2); padding (-inf) adds 0
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < kPartVec; ++i) {
    const float e[4] = {x[i].x, x[i].y, x[i].z, x[i].w};
#pragma unroll
    for (int c = 0; c < 4; ++c)
      sum += __builtin_amdgcn_exp2f(fmaf(e[c], kLog2e, -M2));
  }
  const double wsd = wave_sum((double)sum);
  if (lane == 0) wsum[wave] = wsd;

  // Selection bound: the K-th largest group maximum (with multiplicity).
  // K groups hold an element >= it, so every element of the piece's best K
  // is >= it.  Thread t counts, for group t/4, the group maxima above and
  // at-or-above it in a quarter of the table; a group whose value has fewer
  // than K maxima above and at least K at-or-above is the K-th.
  {
    constexpr int NG = kPartThreads / 4, QG = NG / 4;
    const float z = gz[tid >> 2];
    const float4* g4 = reinterpret_cast<const float4*>(gz + (tid & 3) * QG);
    int gt = 0, ge = 0;
#pragma unroll
    for (int j = 0; j < QG / 4; ++j) {
      const float4 g = g4[j];
      gt += (g.x > z) + (g.y > z) + (g.z > z) + (g.w > z);
      ge += (g.x >= z) + (g.y >= z) + (g.z >= z) + (g.w >= z);
    }
    gt += dpp_i<kDppXor1>(gt);
    gt += dpp_i<kDppXor2>(gt);
    ge += dpp_i<kDppXor1>(ge);
    ge += dpp_i<kDppXor2>(ge);
    if ((tid & 3) == 0 && gt <= a.K - 1 && ge >= a.K) s_tz = z;  // one value
  }
  __syncthreads();
  if (tid == 0) {
    double tot = 0.0;
#pragma unroll
    for (int w = 0; w < kPartThreads / kWave; ++w) tot += wsum[w];
    a.pm[(int64_t)row * a.parts + part] = M2;
    a.ps[(int64_t)row * a.parts + part] = tot;
  }
  float tz = s_tz;
  int tv = 0x7fffffff;
  // -inf: fewer than K groups hold data (a tiny piece); take everything
  bool all = tz == neg_inf();

  // ballot-compacted append of the lanes with `take` to the LDS buffer
  auto offer = [&](float z, int v, bool take) __attribute__((always_inline)) {
    const uint64_t bal = __ballot(take);
    if (bal == 0) return;
    int base = 0;
    if (lane == 0) base = atomicAdd(&s_count, __popcll(bal));
    base = __builtin_amdgcn_readfirstlane(base);
    if (take) {
      const int pos =
          base + __builtin_amdgcn_mbcnt_hi(
                     (uint32_t)(bal >> 32),
                     __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
      if (pos < kPartCap) ck[pos] = zv_key(z, v);
    }
  };
  // common case: collect every element >= the bound from registers (the
  // bound is finite here, so the -inf padding never qualifies)
  if (!all) {
    // a fresh copy of the token base keeps the compiler from computing the
    // token numbers early and holding them across the phases above
    int vc = 4 * (b4 + tid);
    asm volatile("" : "+v"(vc));
#pragma unroll
    for (int i = 0; i < kPartVec; ++i) {
      const int v0 = vc + 4 * kPartThreads * i;
      const float e[4] = {x[i].x, x[i].y, x[i].z, x[i].w};
#pragma unroll
      for (int c = 0; c < 4; ++c) offer(e[c], v0 + c, e[c] >= tz);
    }
  }
  __syncthreads();
  int count = s_count;
  if (all || count > kPartCap) {
    // rare: a tiny piece (take everything) or an overflowing buffer.  The
    // piece is read again from memory, with the bound tightened on each
    // overflow to the K-th best (logit desc, token asc) of the kept
    // elements: at least kPartCap - K of them drop out per round.
    for (;;) {
      if (count > kPartCap) {
        for (int e = tid; e < kPartCap; e += kPartThreads) {
          const uint64_t key = ck[e];
          int rank = 0;
          for (int j = 0; j < kPartCap; ++j) rank += ck[j] > key;
          if (rank == a.K - 1) {
            s_tz = ordered_to_float((uint32_t)(key >> 32));
            s_tv = 0x7fffffff - (int)(uint32_t)key;
          }
        }
        __syncthreads();
        tz = s_tz;
        tv = s_tv;
        all = false;
      }
      __syncthreads();
      if (tid == 0) s_count = 0;
      __syncthreads();
      // a uniform trip count per wave keeps every lane in the ballots
      for (int j0 = b4 + wave * kWave; j0 < e4; j0 += kPartThreads) {
        const int j4 = j0 + lane;
        const bool ok = j4 < e4;
        const float4 y = L4[ok ? j4 : e4 - 1];
        const float e[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int v = 4 * j4 + c;
          offer(e[c], v,
                ok && (all || e[c] > tz || (e[c] == tz && v <= tv)));
        }
      }
      __syncthreads();
      count = s_count;
      if (count <= kPartCap) break;
    }
  }

  // rank the kept elements (keys are distinct); the first K form the
  // piece's sorted list.  Keys are compared eight at a time from 16-byte
  // LDS reads; the buffer is padded with zero keys, below every real key.
  if (tid < 8) ck[count + tid] = 0;
  __syncthreads();
  const int64_t ob = ((int64_t)row * a.parts + part) * a.K;
  const int nblk = (count + 7) / 8;
  for (int e = tid; e < count; e += kPartThreads) {
    const uint64_t key = ck[e];
    int rank = 0;
    const ulonglong2* c2 = reinterpret_cast<const ulonglong2*>(ck);
    for (int j = 0; j < nblk; ++j) {
      const ulonglong2 k0 = c2[4 * j], k1 = c2[4 * j + 1];
      const ulonglong2 k2 = c2[4 * j + 2], k3 = c2[4 * j + 3];
      rank += (k0.x > key) + (k0.y > key) + (k1.x > key) + (k1.y > key) +
              (k2.x > key) + (k2.y > key) + (k3.x > key) + (k3.y > key);
    }
    if (rank < a.K) {
      a.cz[ob + rank] = ordered_to_float((uint32_t)(key >> 32));
      a.cv[ob + rank] = 0x7fffffff - (int)(uint32_t)key;
    }
  }
  for (int r = count + tid; r < a.K; r += kPartThreads) {
    a.cz[ob + r] = neg_inf();
    a.cv[ob + r] = 0x7fffffff;
  }
}

__global__ __launch_bounds__(256) void rowmerge_kernel(RowMergeArgs a) {
  __shared__ float mz[kPartMaxParts * kPartMaxK];
  __shared__ int mv[kPartMaxParts * kPartMaxK];
  __shared__ float s_pm[kPartMaxParts];
  __shared__ double s_ps[kPartMaxParts];
  __shared__ float s_lse;
  __shared__ int s_valid;
  const int row = blockIdx.x, tid = threadIdx.x;
  const int n = a.parts * a.K;
  const int64_t ib = (int64_t)row * n;
  if (tid == 0) s_valid = 0;
  if (tid < a.parts) {
    s_pm[tid] = a.pm[(int64_t)row * a.parts + tid];
    s_ps[tid] = a.ps[(int64_t)row * a.parts + tid];
  }
  int nvalid = 0;
  for (int e = tid; e < n; e += 256) {
    mz[e] = a.cz[ib + e];
    mv[e] = a.cv[ib + e];
    nvalid += mv[e] != 0x7fffffff;
  }
  __syncthreads();
  nvalid = wave_sum(nvalid);
  if ((tid & 63) == 0 && nvalid) atomicAdd(&s_valid, nvalid);
  if (tid == 0) {
    float M = neg_inf(), zt = neg_inf();
    for (int p = 0; p < a.parts; ++p) {
      M = fmaxf(M, s_pm[p]);
      zt = fmaxf(zt, mz[p * a.K]);  // each piece's best logit comes first
    }
    double tot = 0.0;
    for (int p = 0; p < a.parts; ++p)
      if (s_pm[p] != neg_inf()) tot += s_ps[p] * exp2((double)s_pm[p] - M);
    // the row maximum bounds the log-normaliser from below; the log2-domain
    // merge can land an ulp under it on a near one-hot row
    s_lse = fmaxf((float)(kLn2 * ((double)M + log2(tot))), zt);
  }
  __syncthreads();
  const float lse = s_lse;
  const int64_t ob = (int64_t)row * a.kstride;
  for (int e = tid; e < n; e += 256) {
    const float z = mz[e];
    const int v = mv[e];
    if (v == 0x7fffffff) continue;
    const int p = e / a.K;
    int rank = e - p * a.K;
    for (int q = 0; q < a.parts; ++q) {
      if (q == p) continue;
      // entries of list q before (z, v); lists are sorted, padding last
      const float* qz = mz + q * a.K;
      const int* qv = mv + q * a.K;
      int lo = 0, hi = a.K;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (zv_before(qz[mid], qv[mid], z, v))
          lo = mid + 1;
        else
          hi = mid;
      }
      rank += lo;
    }
    if (rank < a.K) {
      a.ltok[ob + rank] = v;
      a.llp[ob + rank] = z - lse;  // log pi
    }
  }
  for (int r = min(s_valid, a.K) + tid; r < a.K; r += 256) {
    a.ltok[ob + r] = -1;
    a.llp[ob + r] = neg_inf();
  }
  if (tid == 0) a.lse[row] = lse;
}

// ---------------------------------------------------------------------

struct BestFirstArgs {
  int B, V, n_max;
  int klist;    // entries per list
  int kstride;  // list row stride
  int truncated;  // lists shorter than the rows they come from
  const int32_t* ltok;
  const float* llp;
  const int32_t* ctx_len;
  int has_cost;
  double C_d, c0, c1, c2, c_ell;
  int32_t *tok, *parent, *depth;
  float* score;
  int32_t* n_star;
  double *phi, *thr;
  int32_t* flag;
  int slow;  // 0: every request, set flag when the lists are too short;
             // 1: only flagged requests
};

// Frontier key, ascending = best-first order: (score desc, parent output
// index asc, child rank asc).  [63:32] inverted ordered score, [31:21]
// parent output index + 1, [20:0] child rank.
__device__ __forceinline__ uint64_t bf_key(float s, int pout, int rank) {
  return ((uint64_t)(~float_to_ordered(s)) << 32) |
         ((uint64_t)(uint32_t)(pout + 1) << 21) | (uint64_t)(uint32_t)rank;
}
__device__ __forceinline__ int bf_pout(uint64_t k) {
  return (int)((k >> 21) & 0x7ff) - 1;
}
__device__ __forceinline__ int bf_rank(uint64_t k) {
  return (int)(k & 0x1fffff);
}

__global__ __launch_bounds__(64) void bestfirst_kernel(BestFirstArgs a) {
  __shared__ uint64_t fkey[kFrontierCap];
  __shared__ uint8_t fdep[kFrontierCap];
  __shared__ float osc[1024];  // scores of the nodes taken so far
  const int q = blockIdx.x, lane = threadIdx.x;
  if (a.slow && !a.flag[q]) return;
  const int B = a.B;
  auto lrow = [&](int d) { return (int64_t)(q * B + d - 1) * a.kstride; };
  int head = 0, tail = 0;

  // insert a key keeping fkey[head..tail) ascending (one wave)
  auto insert = [&](uint64_t key, int dep) {
    int below = 0;
    for (int i = head + lane; i < tail; i += kWave) below += fkey[i] < key;
    below = wave_sum(below);
    const int pos = head + below;
    // shift [pos, tail) right by one, last chunk first
    for (int c0 = ((tail - 1 - pos) / kWave) * kWave; c0 >= 0 && tail > pos;
         c0 -= kWave) {
      const int i = pos + c0 + lane;
      uint64_t k = 0;
      uint8_t dd = 0;
      if (i < tail) {
        k = fkey[i];
        dd = fdep[i];
      }
      __builtin_amdgcn_wave_barrier();
      if (i < tail) {
        fkey[i + 1] = k;
        fdep[i + 1] = dd;
      }
      __builtin_amdgcn_wave_barrier();
    }
    if (lane == 0) {
      fkey[pos] = key;
      fdep[pos] = (uint8_t)dep;
    }
    __builtin_amdgcn_wave_barrier();
    ++tail;
  };

  const double ell = a.has_cost ? (double)a.ctx_len[q] : 0.0;
  auto D = [&](double n) {
    return a.C_d + a.c0 + a.c1 * n + a.c2 * n * n + a.c_ell * ell * n;
  };
  int32_t* otok = a.tok + (int64_t)q * a.n_max;
  int32_t* opar = a.parent + (int64_t)q * a.n_max;
  int32_t* odep = a.depth + (int64_t)q * a.n_max;
  float* osco = a.score + (int64_t)q * a.n_max;

  if (a.klist > 0) {
    const float s = 0.0f + a.llp[lrow(1)];
    insert(bf_key(s + 0.0f, -1, 0), 1);
  }
  int n = 0, overflow = 0;
  double Phi = 0.0;
  for (;;) {
    if (tail == head) break;               // no prefix left
    if (n == a.n_max) break;
    if (!a.slow && a.truncated && n >= a.klist) {
      overflow = 1;                        // the next head may lie past the
      break;                               // lists: rebuild from full lists
    }
    if (tail + 2 > kFrontierCap) {
      overflow = 2;
      break;
    }
    const uint64_t hk = fkey[head];
    const int hd = fdep[head];
    const float hs = key_score(hk);
    const double P = exp((double)hs);
    if (a.has_cost) {
      const double g = P * D((double)n) - (1.0 + Phi) * (D((double)n + 1.0) -
                                                        D((double)n));
      if (g <= 0.0) break;
    }
    ++head;
    const int pout = bf_pout(hk), rank = bf_rank(hk);
    const int htok = a.ltok[lrow(hd) + rank];
    if (lane == 0) {
      otok[n] = htok;
      opar[n] = pout;
      odep[n] = hd;
      osco[n] = hs;
      osc[n] = hs;
    }
    __builtin_amdgcn_wave_barrier();
    Phi += P;
    // next sibling (same parent, next rank) and first child
    const float ps = pout < 0 ? 0.0f : osc[pout];
    if (rank + 1 < a.klist) {
      float s = ps + a.llp[lrow(hd) + rank + 1];
      s = s + 0.0f;
      insert(bf_key(s, pout, rank + 1), hd);
    }
    if (hd < B && a.klist > 0) {
      float s = hs + a.llp[lrow(hd + 1)];
      s = s + 0.0f;
      insert(bf_key(s, n, 0), hd + 1);
    }
    ++n;
  }
  if (!a.slow) {
    if (lane == 0) a.flag[q] = overflow;
    if (overflow == 1) return;  // the slow pass writes this request
  }
  for (int i = n + lane; i < a.n_max; i += kWave) {
    otok[i] = -1;
    opar[i] = -1;
    odep[i] = 0;
    osco[i] = neg_inf();
  }
  if (lane == 0) {
    a.n_star[q] = overflow == 2 ? -1 : n;
    a.phi[q] = Phi;
    a.thr[q] = (1.0 + Phi) / (a.has_cost ? D((double)n) : 1.0);
  }
}

// ---------------------------------------------------------------------
// Batched best-first (same order, same stop, no serial frontier).
//
// The first n nodes of the best-first order are the n best prefixes under
// the key (score desc, parent output index asc, child rank asc), and since
// a child never scores above its parent they form a subtree.  With the
// needed length K <= 64 (the first pass, lists of 64), one workgroup per
// request finds them in parallel:
//  1. a threshold: the K-th best score among the single deviations from
//     the greedy chain (chain node of depth d-1, then any listed token at
//     depth d).  Those are K distinct prefixes scoring at least theta, so
//     the K best prefixes all score at least theta;
//  2. every prefix scoring at least theta, level by level: a node's
//     qualifying children are a prefix of its row's sorted list (binary
//     search), placed by a block-wide prefix sum;
//  3. the K-th best score among those by radix select, then the exact rank
//     of each prefix at or above it under the full key (ties resolved
//     through the ancestors: the parent output order is the order of the
//     parents themselves);
//  4. the stop test at every n at once: P_n = exp(s_n) in parallel, Phi_n
//     summed in order (the serial kernel's rounding), g(n) by ballot.
// A request whose enumeration outgrows kBfCap nodes is flagged and rebuilt
// by the serial kernel, as is one whose tree reaches the list length.

constexpr int kBfThreads = 256;
constexpr int kBfMaxK = 64;     // sequence length of the batched pass
constexpr int kBfMaxRows = 64;  // depths whose lists are staged
constexpr int kBfCap = 2048;    // prefixes at or above the threshold

// Inclusive prefix sum over the 64 lanes of a wave on DPP: shifts by 1, 2,
// 4 and 8 lanes within each row of 16, then each row adds the totals of
// the rows before it (row_bcast:15 into rows 1 and 3, row_bcast:31 into
// rows 2 and 3).  Every lane must be active.
__device__ __forceinline__ int wave_inclusive_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);
  return x;
}

// The k-th largest of keys[0..n) (1 <= k <= n), MSB-first radix select over
// 8-bit digits, starting at the digit of the highest bit in which the keys
// differ (the bits above it are common to all of them): kor / kand are
// this thread's OR / AND of the keys it wrote.  hist has 2 x 256 ints
// (alternate passes), oa 8, sel 2.  Every thread of the workgroup takes
// part; the keys must be visible (a barrier after they were written).
__device__ uint32_t bf_kth_largest(const uint32_t* keys, int n, int k,
                                   uint32_t kor, uint32_t kand, int* hist,
                                   int* oa, int* sel) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  kor = (uint32_t)wave_allreduce32((int)kor, [](int x, int y) { return x | y; });
  kand = (uint32_t)wave_allreduce32((int)kand,
                                    [](int x, int y) { return x & y; });
  if (lane == 0) {
    oa[wave] = (int)kor;
    oa[4 + wave] = (int)kand;
  }
  hist[tid] = 0;
  __syncthreads();
  const uint32_t o = (uint32_t)(oa[0] | oa[1] | oa[2] | oa[3]);
  const uint32_t a = (uint32_t)(oa[4] & oa[5] & oa[6] & oa[7]);
  const uint32_t diff = o ^ a;
  if (diff == 0) return a;  // every key is the same
  const int top = 31 - __builtin_clz(diff);
  int shift = (top / 8) * 8;
  uint32_t mask = shift + 8 >= 32 ? 0u : ~((1u << (shift + 8)) - 1u);
  uint32_t prefix = a & mask;
  for (int pass = 0; shift >= 0; shift -= 8, ++pass) {
    int* h = hist + (pass & 1) * 256;
    hist[((pass + 1) & 1) * 256 + tid] = 0;  // the next pass's histogram
    for (int i = tid; i < n; i += kBfThreads) {
      const uint32_t u = keys[i];
      if ((u & mask) == prefix) atomicAdd(&h[(u >> shift) & 255], 1);
    }
    __syncthreads();
    if (tid < kWave) {
      // lane l holds bins 255-4l .. 252-4l, in descending order
      const int b0 = 255 - 4 * lane;
      const int c0 = h[b0], c1 = h[b0 - 1], c2 = h[b0 - 2], c3 = h[b0 - 3];
      const int s = c0 + c1 + c2 + c3;
      const int inc = wave_inclusive_scan(s);
      const int exc = inc - s;
      if (exc < k && k <= inc) {
        int cum = exc, b = b0;
        if (cum + c0 < k) {
          cum += c0;
          b = b0 - 1;
          if (cum + c1 < k) {
            cum += c1;
            b = b0 - 2;
            if (cum + c2 < k) {
              cum += c2;
              b = b0 - 3;
            }
          }
        }
        sel[0] = b;
        sel[1] = k - cum;
      }
    }
    __syncthreads();
    prefix |= (uint32_t)sel[0] << shift;
    mask |= 0xffu << shift;
    k = sel[1];
  }
  return prefix;
}

__global__ __launch_bounds__(kBfThreads) void bestfirst_batched_kernel(
    BestFirstArgs a) {
  __shared__ float lp[kBfMaxRows * kBfMaxK];       // later: T's scores
  __shared__ uint32_t keys[kBfMaxRows * kBfMaxK];  // later: T, its ranks
  // prefixes; entries kBfCap + lane are wave 0's spare slots (below)
  __shared__ float es[kBfCap + kWave];
  __shared__ int16_t epar[kBfCap + kWave];
  __shared__ uint8_t erank[kBfCap + kWave];
  __shared__ uint8_t edep[kBfCap + kWave];
  __shared__ int16_t eout[kBfCap];
  __shared__ float ch[kBfMaxRows + 1];
  __shared__ int hist[512];
  __shared__ int oa[8];
  __shared__ int sel[2];
  __shared__ int tcount, first_stop, s_ne, s_over;
  __shared__ int seq[kBfMaxK];
  __shared__ double pn[kBfMaxK];
  __shared__ double phis[kBfMaxK + 1];
  static_assert(kBfMaxRows * kBfMaxK >= 2 * kBfCap, "key buffer");

  const int q = blockIdx.x, tid = threadIdx.x, lane = tid & 63,
            wave = tid >> 6;
  const int B = a.B, Kl = a.klist;
  const int K = a.truncated ? min(a.n_max, Kl) : a.n_max;  // <= kBfMaxK
  const int64_t rowb = (int64_t)q * B;

  // 1. lists (padded to 64 entries with -inf) and the greedy chain
  for (int i = tid; i < B * kBfMaxK; i += kBfThreads) {
    const int d = i / kBfMaxK, j = i - d * kBfMaxK;
    lp[i] = j < Kl ? a.llp[(rowb + d) * a.kstride + j] : neg_inf();
  }
  __syncthreads();
  if (tid == 0) {
    float s = 0.0f;
    ch[0] = s;
    for (int d = 0; d < B; ++d) {
      s = s + lp[d * kBfMaxK];
      s = s + 0.0f;
      ch[d + 1] = s;
    }
  }
  __syncthreads();
  const int nc = B * Kl;
  uint32_t kor = 0, kand = 0xffffffffu;
  for (int i = tid; i < nc; i += kBfThreads) {
    const int d = i / Kl, j = i - d * Kl;
    float s = ch[d] + lp[d * kBfMaxK + j];
    s = s + 0.0f;
    const uint32_t u = float_to_ordered(s);
    keys[i] = u;
    kor |= u;
    kand &= u;
  }
  __syncthreads();
  float theta = neg_inf();
  if (nc >= K)
    theta = ordered_to_float(
        bf_kth_largest(keys, nc, K, kor, kand, hist, oa, sel));

  // 2. every prefix scoring at least theta, level by level, in wave 0 alone
  // (no workgroup barriers between levels)
  if (wave == 0) {
    int n_e = 0, lb = 0, le = 0;
    bool over = false;
    for (int d = 1; d <= B && !over; ++d) {
      const int npar = d == 1 ? 1 : le - lb;
      if (npar == 0) break;
      const float* row = lp + (d - 1) * kBfMaxK;
      // the level's list, one entry per lane (Kl <= 64): block ends come
      // from it by readlane, large families are written from it
      const float rl = row[lane];
      int base = n_e;
      for (int x0 = 0; x0 < npar; x0 += kWave) {
        const int x = x0 + lane;
        const bool has = x < npar;
        const float sx = !has ? 0.0f : (d == 1 ? 0.0f : es[lb + x]);
        int c = 0;
        if (has) {
          // qualifying children are a prefix of the sorted row: the last
          // entries of its 8-entry blocks locate the block, then the block
          auto pass = [&](float l) {
            float v = sx + l;
            v = v + 0.0f;
            return v >= theta;
          };
          int b = 0;
#pragma unroll
          for (int k = 0; k < 8; ++k)
            b += pass(__builtin_bit_cast(
                     float, __builtin_amdgcn_readlane(
                                __builtin_bit_cast(int, rl), 8 * k + 7)))
                     ? 1
                     : 0;
          c = 8 * b;
          if (b < 8) {
#pragma unroll
            for (int i = 0; i < 7; ++i) c += pass(row[8 * b + i]) ? 1 : 0;
          }
          c = min(c, Kl);
        }
        const int inc = wave_inclusive_scan(c);
        const int tot = __builtin_amdgcn_readlane(inc, 63);
        if (base + tot > kBfCap) {
          over = true;
          break;
        }
        const int pos0 = base + inc - c;
        const int par = d == 1 ? -1 : lb + x;
        auto put = [&](int pos, float s0, float l, int pr, int j) {
          float s = s0 + l;
          s = s + 0.0f;
          es[pos] = s;
          epar[pos] = (int16_t)pr;
          erank[pos] = (uint8_t)j;
          edep[pos] = (uint8_t)d;
        };
        // small families: each lane writes its own children, the level's
        // first four list entries (the same for every lane; also when every
        // block end passes, as with theta = -inf over a list of at most 4
        // entries), four writes with no branch, those past the family into
        // the lane's spare slot; large ones (the chain node of a flat row
        // has up to 64): the whole wave writes one family at a time
#pragma unroll
        for (int j = 0; j < 4; ++j)
          put(c <= 4 && j < c ? pos0 + j : kBfCap + lane, sx,
              __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                            __builtin_bit_cast(int, rl), j)),
              par, j);
        uint64_t big = __ballot(c > 4);
        while (big) {
          const int L = __builtin_ctzll(big);
          big &= big - 1;
          const int cL = __builtin_amdgcn_readlane(c, L);
          const int pL = __builtin_amdgcn_readlane(pos0, L);
          const int rL = __builtin_amdgcn_readlane(par, L);
          const float sL = __builtin_bit_cast(
              float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sx), L));
          if (lane < cL) put(pL + lane, sL, rl, rL, lane);  // cL <= Kl <= 64
        }
        base += tot;
      }
      // this wave's LDS writes land in order before its later reads
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      lb = n_e;
      n_e = base;
      le = n_e;
    }
    if (lane == 0) {
      s_ne = n_e;
      s_over = over ? 1 : 0;
    }
  }
  __syncthreads();
  const int n_e = s_ne;

  int32_t* otok = a.tok + (int64_t)q * a.n_max;
  int32_t* opar = a.parent + (int64_t)q * a.n_max;
  int32_t* odep = a.depth + (int64_t)q * a.n_max;
  float* osco = a.score + (int64_t)q * a.n_max;
  if (s_over) {
    if (tid == 0) a.flag[q] = 1;  // the serial pass builds this request
    return;
  }

  // 3. the Ke best in exact order
  const int Ke = min(K, n_e);
  if (tid == 0) tcount = 0;
  kor = 0;
  kand = 0xffffffffu;
  for (int i = tid; i < n_e; i += kBfThreads) {
    const uint32_t u = float_to_ordered(es[i]);
    keys[i] = u;
    kor |= u;
    kand &= u;
  }
  __syncthreads();
  uint32_t tk = 0;
  if (Ke > 0) tk = bf_kth_largest(keys, n_e, Ke, kor, kand, hist, oa, sel);
  // T = the prefixes at or above the Ke-th best score: their ids in the
  // upper half of the key buffer, their scores in lp (the lists are no
  // longer needed)
  int* tl = reinterpret_cast<int*>(keys + kBfCap);
  float* ts = lp;
  for (int i = tid; i < n_e; i += kBfThreads) {
    if (keys[i] >= tk) {
      const int o = atomicAdd(&tcount, 1);
      tl[o] = i;
      ts[o] = es[i];
    }
  }
  __syncthreads();
  const int nt = tcount;
  int* trank = reinterpret_cast<int*>(keys);  // E's keys are consumed
  for (int t = tid; t < nt; t += kBfThreads) trank[t] = 0;
  __syncthreads();
  // prefix y before prefix x in the best-first order, for equal scores:
  // the parents' order, the root before any other parent
  auto before_tied = [&](int y, int x) {
    for (;;) {
      const int py = epar[y], px = epar[x];
      if (py == px) return erank[y] < erank[x];
      if (py < 0) return true;
      if (px < 0) return false;
      y = py;
      x = px;
      const float sy = es[y], sx = es[x];
      if (sy != sx) return sy > sx;
    }
  };
  {
    // nt ranks, each split over `parts` threads when nt is small
    const int parts = nt > 0 && nt < kBfThreads ? kBfThreads / nt : 1;
    for (int w = tid; w < nt * parts; w += kBfThreads) {
      const int t = w % nt, part = w / nt;
      const int u0 = (int)((int64_t)nt * part / parts);
      const int u1 = (int)((int64_t)nt * (part + 1) / parts);
      const float sx = ts[t];
      int r = 0;
      for (int u = u0; u < u1; ++u) {
        const float sy = ts[u];
        if (sy > sx)
          ++r;
        else if (sy == sx && u != t && before_tied(tl[u], tl[t]))
          ++r;
      }
      if (r) atomicAdd(&trank[t], r);
    }
  }
  __syncthreads();
  for (int t = tid; t < nt; t += kBfThreads)
    if (trank[t] < Ke) seq[trank[t]] = tl[t];
  __syncthreads();

  // 4. the throughput stop over the sequence
  const double ell = a.has_cost ? (double)a.ctx_len[q] : 0.0;
  auto D = [&](double n) {
    return a.C_d + a.c0 + a.c1 * n + a.c2 * n * n + a.c_ell * ell * n;
  };
  if (tid < Ke) {
    const int x = seq[tid];
    eout[x] = (int16_t)tid;
    pn[tid] = exp((double)es[x]);
  }
  __syncthreads();
  if (tid == 0) {
    double phi = 0.0;
    phis[0] = phi;
    for (int n = 0; n < Ke; ++n) {
      phi += pn[n];
      phis[n + 1] = phi;
    }
  }
  __syncthreads();
  if (tid < kWave) {
    bool stop = false;
    if (a.has_cost && lane < Ke) {
      const double n = (double)lane;
      const double g = pn[lane] * D(n) - (1.0 + phis[lane]) * (D(n + 1.0) - D(n));
      stop = g <= 0.0;
    }
    const uint64_t m = __ballot(stop);
    if (lane == 0) first_stop = m ? (int)__builtin_ctzll(m) : Ke;
  }
  __syncthreads();
  int nstar = first_stop;
  if (nstar == Ke) {
    // no stop before the Ke-th node: the tree is exhausted, or the budget
    // is reached, or the next node may lie past the lists
    int64_t size = 0, pw = 1;
    for (int d = 1; d <= B && size <= Ke; ++d) {
      pw *= Kl;
      size += pw;
    }
    if (size <= Ke) {
    } else if (Ke >= a.n_max) {
      nstar = a.n_max;
    } else {
      if (tid == 0) a.flag[q] = 1;
      return;
    }
  }

  for (int n = tid; n < nstar; n += kBfThreads) {
    const int x = seq[n];
    const int d = edep[x];
    otok[n] = a.ltok[(rowb + d - 1) * a.kstride + erank[x]];
    opar[n] = epar[x] < 0 ? -1 : eout[epar[x]];
    odep[n] = d;
    osco[n] = es[x];
  }
  for (int i = nstar + tid; i < a.n_max; i += kBfThreads) {
    otok[i] = -1;
    opar[i] = -1;
    odep[i] = 0;
    osco[i] = neg_inf();
  }
  if (tid == 0) {
    a.flag[q] = 0;
    a.n_star[q] = nstar;
    const double phi = phis[nstar];
    a.phi[q] = phi;
    a.thr[q] = (1.0 + phi) / (a.has_cost ? D((double)nstar) : 1.0);
  }
}

bool bestfirst_batched_ok(int B, int V, int n_max, int klist) {
  const int K = klist < V ? std::min(n_max, klist) : n_max;
  return K >= 1 && K <= kBfMaxK && B >= 1 && B <= kBfMaxRows &&
         klist >= 1 && klist <= kBfMaxK;
}

hipError_t launch_rowsel(const float* L, int rows, int V, int B, int K,
                         int kstride, const int32_t* only_flagged, int vec_ok,
                         float* lse, int32_t* ltok, float* llp,
                         hipStream_t s) {
  RowSelArgs a{L, V, B, K, kstride, only_flagged, vec_ok, lse, ltok, llp};
  hipLaunchKernelGGL(rowsel_kernel, dim3(rows), dim3(kRowThreads), 0, s, a);
  return hipGetLastError();
}

int rowpart_pieces(int V) {
  const int n4 = V / 4;
  const int per = kPartThreads * kPartVec;
  return n4 <= 0 ? 0 : (n4 + per - 1) / per;
}

bool rowpart_ok(int V, int K, int vec_ok) {
  if (!vec_ok || V % 4 != 0 || K < 1 || K > kPartMaxK) return false;
  const int parts = rowpart_pieces(V);
  if (parts < 1 || parts > kPartMaxParts) return false;
  const int n4 = V / 4, chunk4 = (n4 + parts - 1) / parts;
  return (parts - 1) * chunk4 < n4 && chunk4 <= kPartThreads * kPartVec;
}

hipError_t launch_rowpart(const float* L, int rows, int V, int K, int kstride,
                          float* pm, double* ps, float* cz, int32_t* cv,
                          float* lse, int32_t* ltok, float* llp,
                          hipStream_t s) {
  const int parts = rowpart_pieces(V);
  const int n4 = V / 4;
  RowPartArgs a{L, V, K, parts, (n4 + parts - 1) / parts, pm, ps, cz, cv};
  hipLaunchKernelGGL(rowpart_kernel, dim3(rows, parts), dim3(kPartThreads),
                     0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  RowMergeArgs m{K, parts, kstride, pm, ps, cz, cv, lse, ltok, llp};
  hipLaunchKernelGGL(rowmerge_kernel, dim3(rows), dim3(256), 0, s, m);
  return hipGetLastError();
}

hipError_t launch_bestfirst(int batch, int B, int V, int n_max, int klist,
                            int kstride, int truncated, const int32_t* ltok,
                            const float* llp, const int32_t* ctx_len,
                            const double* cost5, int32_t* tok,
                            int32_t* parent, int32_t* depth, float* score,
                            int32_t* n_star, double* phi, double* thr,
                            int32_t* flag, int slow, hipStream_t s) {
  BestFirstArgs a{};
  a.B = B;
  a.V = V;
  a.n_max = n_max;
  a.klist = klist;
  a.kstride = kstride;
  a.truncated = truncated;
  a.ltok = ltok;
  a.llp = llp;
  a.ctx_len = ctx_len;
  a.has_cost = cost5 != nullptr;
  if (cost5) {
    a.C_d = cost5[0];
    a.c0 = cost5[1];
    a.c1 = cost5[2];
    a.c2 = cost5[3];
    a.c_ell = cost5[4];
  }
  a.tok = tok;
  a.parent = parent;
  a.depth = depth;
  a.score = score;
  a.n_star = n_star;
  a.phi = phi;
  a.thr = thr;
  a.flag = flag;
  a.slow = slow;
  if (slow == 2) {
    a.slow = 0;
    hipLaunchKernelGGL(bestfirst_batched_kernel, dim3(batch),
                       dim3(kBfThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL(bestfirst_kernel, dim3(batch), dim3(64), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace pct

namespace pct {

// ---------------------------------------------------------------------
// Throughput stop over an ordered tree (CaDDTree summary, "Method": the
// tree of the first n nodes of a best-first order has throughput
// f(n) = (1 + Phi_n) / D(n); nodes are added while the gain
// g(n) = P_{n+1} D(n) - (1 + Phi_n)(D(n+1) - D(n)) is positive).
// One wave per request.  Every n is tested at once: each lane takes a
// contiguous chunk of the list, the chunk sums of P_i = exp(s_i) are
// prefix-summed across the wave (double), each lane then walks its chunk
// with the exact Phi_n, and n* is the wave minimum of the lanes' first
// non-positive gains.

__device__ __forceinline__ double shfl_up_d(double x, int delta) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const int lo = __shfl_up((int)(uint32_t)u, delta, kWave);
  const int hi = __shfl_up((int)(uint32_t)(u >> 32), delta, kWave);
  return __builtin_bit_cast(double,
                            ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

__global__ __launch_bounds__(64) void stop_scan_kernel(StopArgs a) {
  const int q = blockIdx.x, lane = threadIdx.x;
  const float* sc = a.score + (int64_t)q * a.N;
  // n_star may alias n_avail: read it before anything is written
  const int n = min(max(a.n_avail[q], 0), a.N);
  __builtin_amdgcn_wave_barrier();
  const double ell = a.ctx_len ? (double)a.ctx_len[q] : 0.0;
  auto D = [&](double m) {
    return a.has_cost ? a.C_d + a.c0 + a.c1 * m + a.c2 * m * m +
                            a.c_ell * ell * m
                      : 1.0;
  };
  const int per = (n + kWave - 1) / kWave;
  const int b0 = min(lane * per, n), b1 = min(b0 + per, n);
  double loc = 0.0;
  for (int i = b0; i < b1; ++i) loc += exp((double)sc[i]);
  // inclusive prefix over the lanes
  double inc = loc;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const double o = shfl_up_d(inc, d);
    if (lane >= d) inc += o;
  }
  double Phi = inc - loc;  // Phi at the chunk start
  int first = n;
  double* f = a.f ? a.f + (int64_t)q * (a.N + 1) : nullptr;
  for (int i = b0; i < b1; ++i) {
    const double P = exp((double)sc[i]);
    if (a.has_cost && first == n) {
      const double Di = D((double)i);
      const double g = P * Di - (1.0 + Phi) * (D((double)i + 1.0) - Di);
      if (g <= 0.0) first = i;
    }
    if (f) f[i] = (1.0 + Phi) / D((double)i);
    Phi += P;
  }
  const int ns = a.has_cost ? -wave_max(-first) : n;
  if (f) {
    // the whole list's throughput, repeated past it (a budget above the
    // available nodes builds the same tree)
    const double total = wave_max(lane == kWave - 1 ? inc : -1.0);
    const double fn = (1.0 + total) / D((double)n);
    for (int i = n + lane; i <= a.N; i += kWave) f[i] = fn;
  }
  // Phi(n*) in the same chunked order
  double ps = 0.0;
  for (int i = b0; i < min(b1, ns); ++i) ps += exp((double)sc[i]);
  const double phi = wave_sum(ps);
  if (lane == 0) {
    if (a.n_star) a.n_star[q] = ns;
    if (a.phi) a.phi[q] = phi;
    if (a.thr) a.thr[q] = (1.0 + phi) / D((double)ns);
  }
  if (a.tok) {
    __builtin_amdgcn_wave_barrier();
    for (int i = ns + lane; i < a.N; i += kWave) {
      const int64_t o = (int64_t)q * a.N + i;
      a.tok[o] = -1;
      a.parent[o] = -1;
      a.depth[o] = 0;
      a.score_out[o] = neg_inf();
    }
  }
}

hipError_t launch_stop_scan(int batch, const StopArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(stop_scan_kernel, dim3(batch), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace pct
