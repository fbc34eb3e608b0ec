// k_markov.hip -- planning and dispatch of the fused Markov-logit kernel
// (the MFMA kernel itself is in k_markov_impl.h), and its plain VALU variant.
// The fused Markov-logit kernel of the parent-conditioned
// tree (PCTree article, "straight draft": z_d(p) = L_d + Markov(p) for every
// frontier parent in one batched call, then each parent's log-softmax and
// local top-k).
//
// Markov(p)[v] = U[tok_p] . W[v] is a [P x r] x [r x V] contraction.  The
// kernel computes it on bf16 MFMA (v_mfma_f32_32x32x16_bf16, fp32
// accumulate) in 64-vocab tiles and consumes every logit in registers:
//   z = L[row_p][v] + M[p][v]            (one fp32 add)
//   running max / sum of 2^(z*log2e - c) per (lane, parent)  (log-sum-exp)
//   candidates z >= theta_p kept in a per-(lane, parent) top-k list
// The logit rows are never written back (unless z_out asks for them).
//
// Orientation: the MFMA "A" operand is the W tile (vocab rows), "B" is the
// gathered U rows (parents), so every lane owns one parent column of a
// 32x32 output block and 16 vocab rows of it: per-parent state lives in a
// handful of registers.  Each wave keeps the U rows of its 64 (NB=2) or 32
// (NB=1) parents resident in registers for the whole kernel; the W tile is
// staged through LDS (double-buffered, XOR-swizzled 16-byte chunks) and
// shared by all waves of the workgroup.  A workgroup covers one slice of the
// vocabulary for up to NB*NW*32 parents; slices x parent tiles form the grid.
#include <algorithm>

#include "k_markov_impl.h"

namespace pct {

// Plain VALU variant for fp32 factors, ranks that are not a multiple of 16,
// or no Markov term at all.  Grid: (vocab slice, parent); each thread walks
// a strided part of the slice.
template <int DT>  // 0 = fp32 factors, 1 = bf16 factors, 2 = none
__global__ __launch_bounds__(kSimpleThreads) void markov_topk_simple(K1Args a) {
  extern __shared__ __align__(16) unsigned char smem[];
  ZV* lists = reinterpret_cast<ZV*>(smem);
  __shared__ float red_c[kSimpleThreads / kWave];
  __shared__ float red_s[kSimpleThreads / kWave];
  const int tid = threadIdx.x;
  const int slice = blockIdx.x, p = blockIdx.y;
  const int v0 = slice * a.vslice, v1 = min(v0 + a.vslice, a.V);
  const int tok = a.ptok ? min(max(a.ptok[p], 0), a.V - 1) : 0;
  int64_t row = a.plrow ? a.plrow[p]
                        : (int64_t)(a.group_fp > 0 ? p / a.group_fp : p) *
                                  a.lrow_mul +
                              a.lrow_add;
  row = row < 0 ? 0 : (row >= a.L_rows ? a.L_rows - 1 : row);
  const float* Lrow = a.L ? a.L + row * a.lstride : nullptr;
  float thr = a.theta ? a.theta[p] : neg_inf();
  float cm2 = neg_inf(), ss = 0.f;
  int cnt = 0;
  ZV* lst = lists + tid * a.k;
  for (int v = v0 + tid; v < v1; v += kSimpleThreads) {
    float mv = 0.f;
    if (DT == 0) {
      const float* u = reinterpret_cast<const float*>(a.U) + (int64_t)tok * a.r;
      const float* w = reinterpret_cast<const float*>(a.W) + (int64_t)v * a.r;
      for (int j = 0; j < a.r; ++j) mv = fmaf(u[j], w[j], mv);
    } else if (DT == 1) {
      const uint16_t* u =
          reinterpret_cast<const uint16_t*>(a.U) + (int64_t)tok * a.r;
      const uint16_t* w =
          reinterpret_cast<const uint16_t*>(a.W) + (int64_t)v * a.r;
      for (int j = 0; j < a.r; ++j)
        mv = fmaf(bf16_bits_to_float(u[j]), bf16_bits_to_float(w[j]), mv);
    }
    const float z = (Lrow ? Lrow[v] : 0.f) + mv;
    if (a.z_out) a.z_out[(int64_t)p * a.V + v] = z;
    if (z >= thr) list_insert(lst, a.k, cnt, thr, z, v);
    const float z2 = z * kLog2e;
    if (z2 > cm2) {
      ss *= __builtin_amdgcn_exp2f(cm2 - z2);
      cm2 = z2;
    }
    ss += __builtin_amdgcn_exp2f(fmaf(z, kLog2e, -cm2));
  }
  // block reduction of (max, sum)
  float m2 = wave_max(cm2);
  float sc = (cm2 == neg_inf()) ? 0.f : ss * __builtin_amdgcn_exp2f(cm2 - m2);
  sc = wave_sum(sc);
  const int wv = tid / kWave;
  if ((tid & 63) == 0) {
    red_c[wv] = m2;
    red_s[wv] = sc;
  }
  __syncthreads();
  if (tid == 0) {
    float M = red_c[0];
    for (int i = 1; i < kSimpleThreads / kWave; ++i) M = fmaxf(M, red_c[i]);
    float S = 0.f;
    if (M != neg_inf())
      for (int i = 0; i < kSimpleThreads / kWave; ++i)
        if (red_c[i] != neg_inf())
          S += red_s[i] * __builtin_amdgcn_exp2f(red_c[i] - M);
    a.part_c[(int64_t)slice * a.P + p] = M;
    a.part_s[(int64_t)slice * a.P + p] = S;
  }
  if (cnt > 0) {
    int pos = atomicAdd(&a.gcnt[p], cnt);
    for (int i = 0; i < cnt; ++i) {
      a.gz[(int64_t)p * a.cap + pos + i] = lst[i].z;
      a.gv[(int64_t)p * a.cap + pos + i] = lst[i].v;
    }
  }
}

// ---------------------------------------------------------------------
// planning and launch

static const int kCUs = 256;
static const size_t kLdsPerCU = 160 * 1024 - 256;  // static LDS headroom

K1Plan plan_k1(int P, int V, int r, int k, int uw_dtype, bool has_uw,
               bool allow_mfma, int group_fp) {
  K1Plan pl{};
  const int R16 = r / 16;
  const bool r_ok = allow_mfma && has_uw && uw_dtype == 1 && r % 16 == 0 &&
                    (R16 == 2 || R16 == 4 || R16 == 8 || R16 == 16);
  if (r_ok) {
    pl.kind = K1_MFMA;
    pl.R16 = R16;
    // At most 32 parents: the thin form, whose eight waves each take their
    // own 32-row pieces of a slice (its LDS holds only the lists).  Slices
    // of whole pieces, one per compute unit.
    const size_t thin_lists = (size_t)kThinWaves * 64 * k * sizeof(ZV);
    if (P <= 32 && thin_lists + 4096 <= kLdsPerCU) {
      pl.thin = 1;
      pl.NB = 1;
      pl.NW = kThinWaves;
      pl.lslots = 0;
      pl.lds = thin_lists;
      pl.lds_total = thin_lists + 2048;
      const int pieces = (V + 31) / 32;
      const int S = std::min(kCUs, pieces);
      pl.vslice = (pieces + S - 1) / S * 32;
      pl.n_slices = (V + pl.vslice - 1) / pl.vslice;
      pl.n_tiles = (V + 63) / 64;
      pl.cap = pl.n_slices * kThinWaves * 2 * k;
      pl.grid = dim3(pl.n_slices, 1);
      pl.block = dim3(kThinWaves * 64);
      return pl;
    }
    // static LDS: two W tiles and two L row buffers; dynamic: the lists
    const size_t wbytes = (size_t)2 * 64 * (2 * R16 + 1) * 16;  // padded rows
    auto slots_of = [&](int nb, int nw) {
      if (group_fp <= 0) return 0;
      const int span = std::min(nw * nb * 32, P);
      return (span + group_fp - 1) / group_fp + 1;
    };
    auto lists_of = [&](int nb, int nw) {  // lists + their lengths
      return (size_t)nw * 64 * nb * (k * sizeof(ZV) + sizeof(int));
    };
    const size_t direct_l = (size_t)2 * 4 * 16 * 16;
    // L bytes of a shape: two buffers of ls row slots of 256 bytes each
    // (ls = 0: rows read directly)
    auto l_bytes = [&](int ls) {
      return ls > 0 ? (size_t)2 * ls * 16 * 16 : direct_l;
    };
    // Eight waves (two per SIMD, so that one's epilogue overlaps the other's
    // MFMA chain) in this order of preference:
    //   64 parents per wave, L rows staged in LDS (more than 256 parents);
    //   32 parents per wave, staged L rows (36 slots, or 16 beside long
    //   lists);
    //   32 parents per wave, L rows read directly (large k, or groups too
    //   small for the row slots).
    // Measured at 640 parents with k = 20: 105 us against 362 us for two
    // waves of 64 parents; at 128 parents of one L row each: 51 against
    // 172 us for one-wave workgroups.  Waves past the parents only load
    // their share of each tile: with few parents the launch is bound by
    // the tile loads, and eight waves issue them faster than one.
    auto fits = [&](int nb, int ls) {
      if (ls > 0 && (group_fp <= 0 || slots_of(nb, 8) > ls)) return false;
      return wbytes + l_bytes(ls) + lists_of(nb, 8) <= kLdsPerCU;
    };
    auto take = [&](int nb, int nw, int ls) {
      pl.NB = nb;
      pl.NW = nw;
      pl.lslots = ls;
      pl.lds = lists_of(nb, nw);
      pl.lds_total = wbytes + l_bytes(ls) + pl.lds;
    };
    if (P > 256 && fits(2, kLdsRowSlots)) {
      take(2, 8, kLdsRowSlots);
    } else if (fits(1, kLdsRowSlots)) {
      take(1, 8, kLdsRowSlots);
    } else if (fits(1, kSmallRowSlots)) {
      take(1, 8, kSmallRowSlots);
    } else if (fits(1, 0)) {
      take(1, 8, 0);
    } else {
      // very long lists: fewer waves of 64 parents, L rows read directly
      int nw = 4;
      while (nw > 1 && wbytes + direct_l + lists_of(2, nw) > kLdsPerCU)
        nw /= 2;
      take(2, nw, 0);
    }
    int per_cu = (int)(kLdsPerCU / pl.lds_total);
    if (per_cu < 1) per_cu = 1;
    const int by_waves = 8 / pl.NW > 0 ? 8 / pl.NW : 1;
    if (per_cu > by_waves) per_cu = by_waves;
    const int PT = (P + 32 * pl.NB * pl.NW - 1) / (32 * pl.NB * pl.NW);
    pl.n_tiles = (V + 63) / 64;
    if (pl.NB == 2) {
      // 64 parents per wave, where the tiles are bound by the MFMA chain
      // and the epilogue: the workgroups of a parent tile take vocabulary
      // tiles from a queue, so as many as the chip holds at once share the
      // tiles and the fastest take the most (a slice is the set of tiles
      // one workgroup took).  Measured at 512 parents: 48.1 -> 45.3 us.
      int S = kCUs * per_cu / PT;
      if (S > pl.n_tiles) S = pl.n_tiles;
      if (S < 1) S = 1;
      pl.n_slices = S;
      pl.tiles_per_slice = 0;
      pl.n_tq = 2 * PT;
    } else {
      // fewer parents per wave, where the tiles are bound by their loads:
      // contiguous slices (the queued order measured 33.8 -> 39.4 us at 256
      // parents)
      int S = (kCUs * per_cu + PT - 1) / PT;
      if (S > pl.n_tiles) S = pl.n_tiles;
      if (S < 1) S = 1;
      pl.tiles_per_slice = (pl.n_tiles + S - 1) / S;
      pl.n_slices = (pl.n_tiles + pl.tiles_per_slice - 1) / pl.tiles_per_slice;
      pl.n_tq = 0;
    }
    pl.cap = pl.n_slices * 2 * k;
    pl.grid = dim3(pl.n_slices, PT);
    pl.block = dim3(pl.NW * 64);
  } else {
    pl.kind = K1_SIMPLE;
    pl.R16 = 0;
    int S = (2048 + P - 1) / P;
    const int max_s = (V + kSimpleThreads - 1) / kSimpleThreads;
    if (S > max_s) S = max_s;
    if (S < 1) S = 1;
    pl.vslice = (V + S - 1) / S;
    pl.n_slices = (V + pl.vslice - 1) / pl.vslice;
    pl.cap = pl.n_slices * kSimpleThreads * k;
    pl.lds = (size_t)kSimpleThreads * k * sizeof(ZV);
    pl.grid = dim3(pl.n_slices, P);
    pl.block = dim3(kSimpleThreads);
  }
  return pl;
}

#define PCT_DECL_RANK(R)                                                  \
  hipError_t launch_mfma_r##R##s(const K1Plan&, const K1Args&, hipStream_t); \
  hipError_t launch_mfma_r##R##d(const K1Plan&, const K1Args&, hipStream_t);
PCT_DECL_RANK(2)
PCT_DECL_RANK(4)
PCT_DECL_RANK(8)
PCT_DECL_RANK(16)
#undef PCT_DECL_RANK

template <int DT>
static hipError_t go_simple(const K1Plan& pl, const K1Args& a,
                            hipStream_t s) {
  auto fn = markov_topk_simple<DT>;
  hipError_t e = allow_lds(reinterpret_cast<const void*>(fn), pl.lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fn, pl.grid, pl.block, pl.lds, s, a);
  return hipGetLastError();
}

__global__ void fill_i32_kernel(int32_t* p, int n, int32_t v) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}

hipError_t launch_fill_i32(int32_t* p, int n, int32_t v, hipStream_t s) {
  hipLaunchKernelGGL(fill_i32_kernel, dim3((n + 255) / 256), dim3(256), 0, s,
                     p, n, v);
  return hipGetLastError();
}

hipError_t launch_k1(const K1Plan& pl, const K1Args& a, hipStream_t s) {
  if (pl.kind == K1_MFMA) {
    // the queued order is compiled into the kernels of two parent blocks
    // per wave
    if ((pl.NB == 2) != (pl.n_tq > 0) || (pl.n_tq > 0 && a.tq == nullptr))
      return hipErrorInvalidValue;
    const bool st = !pl.thin && a.group_fp > 0 && a.lslots > 0 &&
                    a.vec_ok && a.L != nullptr && a.plrow == nullptr;
    switch (pl.R16) {
      case 2: return st ? launch_mfma_r2s(pl, a, s) : launch_mfma_r2d(pl, a, s);
      case 4: return st ? launch_mfma_r4s(pl, a, s) : launch_mfma_r4d(pl, a, s);
      case 8: return st ? launch_mfma_r8s(pl, a, s) : launch_mfma_r8d(pl, a, s);
      case 16:
        return st ? launch_mfma_r16s(pl, a, s) : launch_mfma_r16d(pl, a, s);
    }
    return hipErrorInvalidValue;
  }
  if (a.U == nullptr) return go_simple<2>(pl, a, s);
  if (a.dt == 1) return go_simple<1>(pl, a, s);
  return go_simple<0>(pl, a, s);
}

}  // namespace pct
