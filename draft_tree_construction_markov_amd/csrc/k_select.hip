// k_select.hip -- per-request selection kernels of the parent-conditioned
// tree (PCTree article, "chain -> tree"): merging the per-slice partials of
// the fused Markov kernel into each parent's log-normaliser and local top-k,
// path scores s(c) = s(p) + log pi(c|p), the per-depth beam (top-k pruning
// at each stage), and the global top-N that fits the verify budget.  Also
// the threshold seeds that let the fused kernel skip almost every logit.
#include "pct_device.h"
#include "pct_internal.h"

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

// Per L row, the kSeedT tokens of largest L: each thread keeps its best
// element, then the workgroup keeps the kSeedT best of those (any subset is
// a valid seed; this one is nearly the row's top kSeedT).
__global__ __launch_bounds__(256) void row_top_kernel(const float* L, int V,
                                                       int64_t lstride,
                                                       int vec_ok,
                                                       int32_t* rowtop) {
  __shared__ float sz[256];
  __shared__ int32_t sv[256];
  const int row = blockIdx.x, tid = threadIdx.x;
  const float* Lr = L + (int64_t)row * lstride;
  float bz = neg_inf();
  int32_t bv = 0x7fffffff;
  if (vec_ok) {
    const float4* L4 = reinterpret_cast<const float4*>(Lr);
    const int n4 = V / 4;
    for (int i = tid; i < n4; i += 256) {
      const float4 x = L4[i];
      const int v = 4 * i;
      if (zv_before(x.x, v, bz, bv)) { bz = x.x; bv = v; }
      if (zv_before(x.y, v + 1, bz, bv)) { bz = x.y; bv = v + 1; }
      if (zv_before(x.z, v + 2, bz, bv)) { bz = x.z; bv = v + 2; }
      if (zv_before(x.w, v + 3, bz, bv)) { bz = x.w; bv = v + 3; }
    }
    for (int v = 4 * n4 + tid; v < V; v += 256)
      if (zv_before(Lr[v], v, bz, bv)) { bz = Lr[v]; bv = v; }
  } else {
    for (int v = tid; v < V; v += 256)
      if (zv_before(Lr[v], v, bz, bv)) { bz = Lr[v]; bv = v; }
  }
  sz[tid] = bz;
  sv[tid] = bv;
  // slots without a distinct token (V < kSeedT) stay -1 and are skipped
  if (tid < kSeedT) rowtop[(int64_t)row * kSeedT + tid] = -1;
  __syncthreads();
  int rank = 0;
  for (int j = 0; j < 256; ++j) rank += zv_before(sz[j], sv[j], bz, bv);
  if (rank < kSeedT && bv < V) rowtop[(int64_t)row * kSeedT + rank] = bv;
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
// combined in double.
__device__ float wave_merge_lse(const float* part_c, const float* part_s,
                                int S, int P, int p, int lane) {
  double cm = -__builtin_inf();
  for (int s = lane; s < S; s += kWave) {
    const double c = part_c[(int64_t)s * P + p];
    cm = c > cm ? c : cm;
  }
  cm = wave_max(cm);
  double acc = 0.0;
  for (int s = lane; s < S; s += kWave) {
    const float c = part_c[(int64_t)s * P + p];
    const float v = part_s[(int64_t)s * P + p];
    if (c != neg_inf() && v > 0.f) acc += (double)v * exp2((double)c - cm);
  }
  acc = wave_sum(acc);
  return (float)(kLn2 * (cm + log2(acc)));
}

// The i-th best candidate (z desc, token asc) of a parent, i = 0..k-1, by k
// passes that each take the best entry after the previous pick.  Results on
// every lane.
template <typename F>
__device__ void wave_topk(const float* gz, const int32_t* gv, int cnt, int k,
                          int lane, F&& emit) {
  float pz = pos_inf();
  int32_t pv = -1;
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
    if (bv == 0x7fffffff) bv = 0;  // fewer than k candidates: cannot happen
    emit(i, bz, bv);                // with a valid threshold seed
    pz = bz;
    pv = bv;
  }
}

// ---------------------------------------------------------------------
// Depth-1 frontier: the anchor of each request.
__global__ __launch_bounds__(64) void init_kernel(int B, const int32_t* anchor,
                                                  Frontier f, int32_t* gcnt,
                                                  SeedArgs sa) {
  const int q = blockIdx.x, lane = threadIdx.x;
  const int a = anchor[q];
  const float th = seed_theta(sa, a, q * B, lane);
  if (lane == 0) {
    f.tok[q] = a;
    f.pid[q] = -1;
    f.lrow[q] = q * B;
    f.s[q] = 0.f;
    f.theta[q] = th;
    gcnt[q] = 0;
  }
}

// One workgroup per request: children of every frontier parent, their
// scores and pool keys, the beam of the next depth and its seeds.
__global__ __launch_bounds__(256) void expand_kernel(ExpandArgs a) {
  __shared__ uint64_t ckey[kMaxCand];
  __shared__ int32_t cpid[kMaxCand];
  __shared__ int32_t ntok[kMaxCand];
  const int q = blockIdx.x, tid = threadIdx.x, lane = tid & 63,
            wave = tid >> 6;
  const int NC = a.Fp * a.k;
  for (int j = wave; j < a.Fp; j += 4) {
    const int p = q * a.Fp + j;
    const int sp = a.shared_stats ? q : p;
    const float lse =
        wave_merge_lse(a.part_c, a.part_s, a.n_slices, a.Pstat, sp, lane);
    const float sp_score = a.cur.s[p];
    const int ppid = a.cur.pid[p];
    const int cnt = min(a.gcnt[sp], a.cap);
    wave_topk(a.gz + (int64_t)sp * a.cap, a.gv + (int64_t)sp * a.cap, cnt,
              a.k, lane, [&](int i, float z, int32_t v) {
                if (lane == 0) {
                  const float l = z - lse;       // log pi(v|p)
                  float s = sp_score + l;        // path score
                  s = s + 0.0f;                  // -0 -> +0
                  const int pid = a.base_d + j * a.k + i;
                  const uint64_t key = make_key(s, ppid, v);
                  ckey[j * a.k + i] = key;
                  cpid[j * a.k + i] = pid;
                  a.pool_key[(int64_t)q * a.pool_n + pid] = key;
                }
              });
  }
  __syncthreads();
  // beam: the Fn smallest keys of this depth's children, by rank (keys are
  // distinct: (parent, token) pairs are unique)
  for (int c = tid; c < NC; c += 256) {
    const uint64_t key = ckey[c];
    int rank = 0;
    for (int o = 0; o < NC; ++o) rank += ckey[o] < key;
    if (rank < a.Fn) {
      const int o = q * a.Fn + rank;
      a.nxt.tok[o] = key_tok(key);
      a.nxt.pid[o] = cpid[c];
      a.nxt.s[o] = key_score(key);
      a.nxt.lrow[o] = q * a.B + a.d;  // row of depth d+1
      ntok[rank] = key_tok(key);
      if (a.gcnt_next) a.gcnt_next[o] = 0;
    }
  }
  if (a.d >= a.B) return;
  __syncthreads();
  for (int i = wave; i < a.Fn; i += 4) {
    const float th = seed_theta(a.seed, ntok[i], q * a.B + a.d, lane);
    if (lane == 0) a.nxt.theta[q * a.Fn + i] = th;
  }
}

// Global top-N of every generated child of one request, by key; parents
// remapped to output indices.  Bitonic sort in LDS.
__global__ __launch_bounds__(1024) void topn_kernel(TopNArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  int n2 = 1;
  while (n2 < a.pool_n) n2 <<= 1;
  uint64_t* key = reinterpret_cast<uint64_t*>(smem);
  int16_t* id = reinterpret_cast<int16_t*>(smem + 8 * n2);
  int16_t* inv = id + n2;
  const int q = blockIdx.x, tid = threadIdx.x;
  for (int i = tid; i < n2; i += 1024) {
    key[i] = i < a.pool_n ? a.pool_key[(int64_t)q * a.pool_n + i]
                          : ~(uint64_t)0;
    id[i] = (int16_t)i;
    inv[i] = -1;
  }
  __syncthreads();
  for (int size = 2; size <= n2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < n2 / 2; i += 1024) {
        const int lo = 2 * stride * (i / stride) + (i % stride);
        const int hi = lo + stride;
        const bool up = (lo & size) == 0;
        const uint64_t kl = key[lo], kh = key[hi];
        if ((kl > kh) == up) {
          key[lo] = kh;
          key[hi] = kl;
          const int16_t t = id[lo];
          id[lo] = id[hi];
          id[hi] = t;
        }
      }
      __syncthreads();
    }
  }
  const int n = min(a.N, a.pool_n);
  for (int i = tid; i < n; i += 1024) inv[id[i]] = (int16_t)i;
  __syncthreads();
  for (int i = tid; i < a.N; i += 1024) {
    const int64_t o = (int64_t)q * a.N + i;
    if (i < n) {
      const uint64_t k = key[i];
      const int pid = id[i];
      int d = 1;
      while (d < a.B && pid >= a.base[d + 1]) ++d;
      const int pp = key_ppid(k);
      a.tok[o] = key_tok(k);
      a.parent[o] = pp < 0 ? -1 : inv[pp];
      a.depth[o] = d;
      a.score[o] = key_score(k);
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
  const float lse = wave_merge_lse(part_c, part_s, S, P, p, lane);
  const int cnt = min(gcnt[p], cap);
  wave_topk(gz + (int64_t)p * cap, gv + (int64_t)p * cap, cnt, k, lane,
            [&](int i, float z, int32_t v) {
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
  hipLaunchKernelGGL(row_top_kernel, dim3(rows), dim3(256), 0, s, L, V,
                     lstride, vec_ok, rowtop);
  return hipGetLastError();
}

hipError_t launch_init(int batch, int B, const int32_t* anchor, Frontier f,
                       int32_t* gcnt, const SeedArgs& sa, hipStream_t s) {
  hipLaunchKernelGGL(init_kernel, dim3(batch), dim3(64), 0, s, B, anchor, f,
                     gcnt, sa);
  return hipGetLastError();
}

hipError_t launch_expand(const ExpandArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(expand_kernel, dim3(a.batch), dim3(256), 0, s, a);
  return hipGetLastError();
}

size_t topn_lds(int pool_n) {
  int n2 = 1;
  while (n2 < pool_n) n2 <<= 1;
  return (size_t)n2 * 12;
}

hipError_t launch_topn(const TopNArgs& a, hipStream_t s) {
  hipError_t e = allow_lds(reinterpret_cast<const void*>(topn_kernel),
                           topn_lds(a.pool_n));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topn_kernel, dim3(a.batch), dim3(1024),
                     topn_lds(a.pool_n), s, a);
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
