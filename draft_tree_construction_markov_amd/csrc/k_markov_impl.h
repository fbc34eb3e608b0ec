// k_markov_impl.h -- the fused Markov-logit kernel of the parent-conditioned
// tree (PCTree article, "straight draft": z_d(p) = L_d + Markov(p) for every
// frontier parent in one batched call, then each parent's log-softmax and
// local top-k).
//
// Markov(p)[v] = U[tok_p] . W[v] is a [P x r] x [r x V] contraction.  The
// kernel computes it on bf16 MFMA (v_mfma_f32_32x32x16_bf16, fp32
// accumulate) in 64-vocab tiles and consumes every logit in registers:
//   z = L[row_p][v] + M[p][v]            (one fp32 add)
//   sum of 2^(z*log2e - c) per (lane, parent)  (log-sum-exp; the tiled
//   kernel fixes the shift c just below the parent's threshold, the thin
//   form keeps a running maximum)
//   candidates z >= theta_p kept in a per-(lane, parent) top-k list
// The logit rows are never written back (unless z_out asks for them).
//
// Orientation: the MFMA "A" operand is the W tile (vocab rows), "B" is the
// gathered U rows (parents), so every lane owns one parent column of a
// 32x32 output block and 16 vocab rows of it: per-parent state lives in a
// handful of registers.  Each wave keeps the U rows of its 64 (NB=2) or 32
// (NB=1) parents resident in registers for the whole kernel; the W tile is
// staged through LDS by direct global->LDS loads (double-buffered, rows
// padded by one 16-byte chunk) and shared by all waves of the workgroup;
// so are the workgroup's L rows when parents are grouped by request.  A
// workgroup covers a slice of the vocabulary for up to NB*NW*32 parents;
// slices x parent tiles form the grid.  With 64 parents per wave a slice is
// the set of 64-row tiles the workgroup took from a queue shared by the
// workgroups of its parent tile; otherwise it is a contiguous run of tiles.
#pragma once
#include "pct_device.h"
#include "pct_internal.h"

namespace pct {

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef const __attribute__((address_space(1))) void* gbl_ptr_t;

// W tile layout in LDS: 64 rows of 2*R16 16-byte chunks, each row followed
// by one pad chunk (row stride 2*R16 + 1 chunks).  The pad spreads the rows
// of one MFMA operand read over all LDS banks, and chunk (row, c) sits at
// row * stride + c, so a lane's reads of one tile differ only by immediate
// offsets from one base address (no address register per rank step).
template <int R16>
constexpr int wstride() {
  return 2 * R16 + 1;
}

// Insert z (vocab v) into a lane's top-k list: the list keeps the k largest
// elements offered, an equal logit ranking the smaller vocabulary index
// first, whatever the order in which they come (a workgroup's tiles arrive
// in queue order).
__device__ __forceinline__ void list_insert(ZV* lst, int k, int& cnt,
                                            float& thr, float z, int v) {
  if (cnt < k) {
    lst[cnt] = ZV{z, v};
    ++cnt;
    if (cnt == k) {
      float mn = lst[0].z;
      for (int i = 1; i < k; ++i) mn = fminf(mn, lst[i].z);
      thr = mn;
    }
  } else if (z >= thr) {
    int wi = 0;
    float wz = lst[0].z;
    int wv = lst[0].v;
    for (int i = 1; i < k; ++i) {
      ZV e = lst[i];
      if (e.z < wz || (e.z == wz && e.v > wv)) {
        wi = i;
        wz = e.z;
        wv = e.v;
      }
    }
    if (z == wz && v > wv) return;
    lst[wi] = ZV{z, v};
    float mn = lst[0].z;
    for (int i = 1; i < k; ++i) mn = fminf(mn, lst[i].z);
    thr = mn;
  }
}

__device__ __forceinline__ void flush_lane(const K1Args& a, int p, int slice,
                                           float c2, float s, ZV* lst,
                                           int cnt, bool writer) {
  if (writer) {
    a.part_c[(int64_t)slice * a.P + p] = c2;
    a.part_s[(int64_t)slice * a.P + p] = s;
  }
  if (cnt > 0) {
    int pos = atomicAdd(&a.gcnt[p], cnt);
    float* gz = a.gz + (int64_t)p * a.cap + pos;
    int32_t* gv = a.gv + (int64_t)p * a.cap + pos;
    for (int i = 0; i < cnt; ++i) {
      gz[i] = lst[i].z;
      gv[i] = lst[i].v;
    }
  }
}

// Combine the (max, sum) partials of lanes l and l^32 (same parent).
__device__ __forceinline__ void combine_halves(float& c2, float& s, int lane) {
  float oc2 = swap_halves(c2, lane);
  float os = swap_halves(s, lane);
  float m2 = fmaxf(c2, oc2);
  float r = 0.f;
  if (m2 != neg_inf()) {
    if (c2 != neg_inf()) r += s * __builtin_amdgcn_exp2f(c2 - m2);
    if (oc2 != neg_inf()) r += os * __builtin_amdgcn_exp2f(oc2 - m2);
  }
  c2 = m2;
  s = r;
}

// value of x in lane g of this lane's quad (a DPP quad_perm source operand)
__device__ __forceinline__ float quad_bcast(float x, int g) {
  const int xi = __builtin_bit_cast(int, x);
  int r;
  switch (g) {
    case 0: r = __builtin_amdgcn_mov_dpp(xi, 0x00, 0xf, 0xf, true); break;
    case 1: r = __builtin_amdgcn_mov_dpp(xi, 0x55, 0xf, 0xf, true); break;
    case 2: r = __builtin_amdgcn_mov_dpp(xi, 0xaa, 0xf, 0xf, true); break;
    default: r = __builtin_amdgcn_mov_dpp(xi, 0xff, 0xf, 0xf, true); break;
  }
  return __builtin_bit_cast(float, r);
}

template <int NB, int NW, int R16, bool STAGED, int LSL = kLdsRowSlots>
__global__ __launch_bounds__(NW * 64) void markov_topk_mfma(K1Args a) {
  constexpr int CH = 2 * R16;               // 16-byte chunks per W row
  constexpr int RS = wstride<R16>();       // chunks per padded LDS row
  constexpr int TILE_CH = 64 * RS;          // chunk slots per 64-row tile
  constexpr int SPAN = NW * NB * 32;        // parents per workgroup
  constexpr int LS = STAGED ? LSL : 4;  // L row slots per buffer
  // Double buffers as distinct LDS objects: the loop is unrolled by two so
  // that every read names one buffer and every direct global->LDS load the
  // other, which lets the compiler keep the next tile's loads in flight
  // while the current tile is read (no conservative wait on aliasing).
  __shared__ __align__(16) uint4 w0[TILE_CH];
  __shared__ __align__(16) uint4 w1[TILE_CH];
  __shared__ __align__(16) float4 l0[LS * 16];
  __shared__ __align__(16) float4 l1[LS * 16];
  extern __shared__ __align__(16) unsigned char smem[];
  ZV* lists = reinterpret_cast<ZV*>(smem);
  // per (lane, parent) list lengths live in LDS: only the rare path uses them
  int* lcount = reinterpret_cast<int*>(lists + NW * 64 * NB * a.k);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, col = lane & 31;
  const int slice = blockIdx.x;
  const int nwg = gridDim.x;
  // Tile order.  Without a queue, workgroup s takes the contiguous tiles
  // t0 .. t1-1 of its slice.  With one (two counters per parent tile:
  // tickets handed out, workgroups finished), its tiles 0 and 1 are s and
  // s + nwg and tile i >= 2 is 2*nwg plus a ticket taken during tile i - 2,
  // so the workgroups that run fastest take the most tiles; their ids pass
  // through the ring sq[i % 4].  An id past the last tile ends the loop.
  // (the shapes of 64 parents per wave use the queue; the planner gives
  // their launches one)
  constexpr bool queued = NB == 2;
  int32_t* tq = queued ? a.tq + 2 * blockIdx.y : nullptr;
  const int t0 = queued ? slice : slice * a.tiles_per_slice;
  const int t1 =
      queued ? a.n_tiles : min(t0 + a.tiles_per_slice, a.n_tiles);
  auto fixed_id = [&](int i) __attribute__((always_inline)) {
    const int t = queued ? slice + i * nwg : t0 + i;
    return t < t1 ? t : a.n_tiles;
  };
  __shared__ int sq[4];
  const int p0 = blockIdx.y * SPAN;
  const int pw = p0 + wave * (NB * 32);
  const bool has_L = a.L != nullptr;
  const uint4* Wg = reinterpret_cast<const uint4*>(a.W);
  // grouped rows of this workgroup: groups g0 .. g0 + nslots - 1
  const int g0 = STAGED ? p0 / a.group_fp : 0;
  const int nslots =
      STAGED ? (min(p0 + SPAN, a.P) - 1) / a.group_fp - g0 + 1 : 0;

  // quads of lanes share one L row when groups are whole quads
  const bool quadL = STAGED && (a.group_fp & 3) == 0 && (a.P & 3) == 0;
  bf16x8 uf[NB][R16];
  const float* lrow[NB];
  int lslot[NB];
  float thr[NB], cm2[NB], ss[NB], hb[NB];
  // per-parent scalars first: a wait for any of them (vmcnt counts in
  // order) then cannot hold up the fragment loads issued after them
  int ptk[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int p = pw + 32 * b + col;
    const bool valid = p < a.P;
    const int pc = valid ? p : a.P - 1;
    ptk[b] = a.upack != nullptr ? 0 : min(max(a.ptok[pc], 0), a.V - 1);
    lcount[(wave * 64 + lane) * NB + b] = 0;
    int64_t row = a.plrow ? a.plrow[pc]
                          : (int64_t)(a.group_fp > 0 ? pc / a.group_fp : pc) *
                                    a.lrow_mul +
                                a.lrow_add;
    row = row < 0 ? 0 : (row >= a.L_rows ? a.L_rows - 1 : row);
    lrow[b] = (!STAGED && has_L) ? a.L + row * a.lstride : nullptr;
    lslot[b] = STAGED ? pc / a.group_fp - g0 : 0;
    thr[b] = valid ? (a.theta ? a.theta[p] : neg_inf()) : pos_inf();
    // the exponent shift of the lane's sum: fixed just below the threshold
    // (+inf past the parents, whose sums stay 0)
    cm2[b] = valid ? thr[b] * kLog2e - 1.f : pos_inf();
    ss[b] = 0.f;
    hb[b] = 1.f;
  }
  // The fragment loads are unconditional and in bounds (a block past the
  // parents reads block 0; the packed buffer holds whole blocks), so that
  // they and the first tile's loads are in flight together; fragments of
  // parents past P are zeroed once both have arrived.
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    if (a.upack != nullptr) {
      // packed rows: one contiguous 1 KB load per rank step
      const int blk = pw + 32 * b < a.P ? (pw + 32 * b) >> 5 : 0;
      const uint4* up = a.upack + (int64_t)blk * R16 * 64 + lane;
#pragma unroll
      for (int kk = 0; kk < R16; ++kk)
        uf[b][kk] = __builtin_bit_cast(bf16x8, up[kk * 64]);
    } else {
      const uint4* up =
          reinterpret_cast<const uint4*>(a.U) + (int64_t)ptk[b] * CH + h;
#pragma unroll
      for (int kk = 0; kk < R16; ++kk)
        uf[b][kk] = __builtin_bit_cast(bf16x8, up[2 * kk]);
    }
  }

  // Tile t -> LDS by direct global->LDS loads.  W: each wave instruction
  // fills 64 consecutive 16-byte slots; slot q holds row q/RS, chunk q%RS
  // (the pad chunk q%RS == CH receives a copy of the row's chunk 0, never
  // read).  Rows past V are clamped to row V-1 (their outputs are masked).  L (staged):
  // 16 chunks per row slot; V % 4 == 0 here, so a chunk is inside the row or
  // wholly past V (then an in-bounds dummy that is never read).
  constexpr int LMAX = (LS * 16 + 64 * NW - 1) / (64 * NW);  // L DMAs/wave
  auto issue = [&](int t, uint4* wd, float4* ld) __attribute__((always_inline)) {
    // L sources first: any register reload happens before DMAs are in
    // flight, so it cannot make the wave wait for them
    const float* lsrc[LMAX];
    if (STAGED) {
#pragma unroll
      for (int i = 0; i < LMAX; ++i) {
        const int c = (wave + i * NW) * 64 + lane;
        const int slot = min(c >> 4, nslots - 1);
        int64_t row = (int64_t)(g0 + slot) * a.lrow_mul + a.lrow_add;
        row = row >= a.L_rows ? a.L_rows - 1 : row;
        int v = 64 * t + 4 * (c & 15);
        if (v >= a.V) v = 0;
        lsrc[i] = a.L + row * a.lstride + v;
      }
    }
    const uint4* wbase = Wg + (int64_t)64 * t * CH;
    const bool wfull = 64 * t + 64 <= a.V;
#pragma unroll
    for (int gi = wave; gi < TILE_CH / 64; gi += NW) {
      const int q = gi * 64 + lane;
      int row = q / RS;
      int c = q - row * RS;
      c = c < CH ? c : 0;
      if (!wfull && 64 * t + row >= a.V) row = a.V - 1 - 64 * t;
      const int off = row * CH + c;
      __builtin_amdgcn_global_load_lds((gbl_ptr_t)(wbase + off),
                                       (lds_ptr_t)(wd + gi * 64), 16, 0, 0);
    }
    // L rows non-temporal (aux 2): each is read once per launch, while W
    // is read again by every depth and should stay in the caches.  The LDS
    // destinations are per-wave values, derived from a scalar copy of the
    // wave index so that none of them occupies a vector register.
    if (STAGED) {
      const int ws = __builtin_amdgcn_readfirstlane(wave);
#pragma unroll
      for (int i = 0; i < LMAX; ++i) {
        const int gi = ws + i * NW;
        if (gi * 64 < nslots * 16)
          __builtin_amdgcn_global_load_lds((gbl_ptr_t)lsrc[i],
                                           (lds_ptr_t)(ld + gi * 64), 16, 0,
                                           2);
      }
    }
  };

  f32x16 acc[NB];
  // MFMA chain of half av of the tile in wt: acc[b] = W rows . U rows.  The
  // A operand of step kk is chunk 2*kk + h of row 32*av + col; its reads run
  // kRA steps ahead of the MFMAs that consume them.
  const int wlane = col * RS + h;
  auto mma = [&](const uint4* wt, int av) __attribute__((always_inline)) {
    constexpr int kRA = R16 < 4 ? R16 : 4;
    const uint4* wp = wt + wlane + 32 * RS * av;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[b][j] = 0.f;
    bf16x8 wf[kRA];
#pragma unroll
    for (int i = 0; i < kRA; ++i) wf[i] = __builtin_bit_cast(bf16x8, wp[2 * i]);
#pragma unroll
    for (int kk = 0; kk < R16; ++kk) {
      const bf16x8 cur = wf[kk % kRA];
      if (kk + kRA < R16)
        wf[kk % kRA] = __builtin_bit_cast(bf16x8, wp[2 * (kk + kRA)]);
#pragma unroll
      for (int b = 0; b < NB; ++b)
        acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, uf[b][kk],
                                                        acc[b], 0, 0, 0);
    }
    // keep the schedule in that order: kRA reads first, then each step's
    // MFMAs followed by the read kRA steps ahead
    __builtin_amdgcn_sched_group_barrier(0x100, kRA, 0);  // LDS reads
#pragma unroll
    for (int kk = 0; kk < R16; ++kk) {
      __builtin_amdgcn_sched_group_barrier(0x008, NB, 0);  // MFMAs
      if (kk + kRA < R16) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  };
  // Epilogue of half av of tile t (L rows of the tile in lt): z = L + acc,
  // running max / exp-sum, rare top-k path.
  auto epi = [&](int t, int av, const float4* lt) __attribute__((always_inline)) {
    const bool full = 64 * t + 64 <= a.V;
    {
      // register j of this lane holds vocab vb + 8*(j/4) + j%4
      const int vb = 64 * t + 32 * av + 4 * h;
      // one L float4 per lane and parent block, all read before the first
      // block's adds
      float4 lq[NB];
      if (STAGED && full && quadL) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
          lq[b] = lt[lslot[b] * 16 + 8 * av + h + 2 * (lane & 3)];
      }
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        float z[16];
        if (STAGED) {
          const float4* lp = lt + lslot[b] * 16 + 8 * av + h;
          if (full && quadL) {
            // the four lanes of a quad hold four consecutive parents of one
            // group, so they need the same 16 L values: each lane reads one
            // float4 and the adds take the others from the quad's lanes
            const float4 l4 = lq[b];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              z[4 * g + 0] = quad_bcast(l4.x, g) + acc[b][4 * g + 0];
              z[4 * g + 1] = quad_bcast(l4.y, g) + acc[b][4 * g + 1];
              z[4 * g + 2] = quad_bcast(l4.z, g) + acc[b][4 * g + 2];
              z[4 * g + 3] = quad_bcast(l4.w, g) + acc[b][4 * g + 3];
            }
          } else if (full) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const float4 l4 = lp[2 * g];
              z[4 * g + 0] = l4.x + acc[b][4 * g + 0];
              z[4 * g + 1] = l4.y + acc[b][4 * g + 1];
              z[4 * g + 2] = l4.z + acc[b][4 * g + 2];
              z[4 * g + 3] = l4.w + acc[b][4 * g + 3];
            }
          } else {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const float4 l4 = lp[2 * g];
              const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
              for (int e = 0; e < 4; ++e)
                z[4 * g + e] = vb + 8 * g + e < a.V ? lv[e] + acc[b][4 * g + e]
                                                     : neg_inf();
            }
          }
        } else if (full && a.vec_ok) {
          if (has_L) {
            const float4* lp = reinterpret_cast<const float4*>(lrow[b] + vb);
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const float4 l4 = lp[2 * g];
              z[4 * g + 0] = l4.x + acc[b][4 * g + 0];
              z[4 * g + 1] = l4.y + acc[b][4 * g + 1];
              z[4 * g + 2] = l4.z + acc[b][4 * g + 2];
              z[4 * g + 3] = l4.w + acc[b][4 * g + 3];
            }
          } else {
#pragma unroll
            for (int j = 0; j < 16; ++j) z[j] = acc[b][j];
          }
        } else {
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int v = vb + 8 * (j >> 2) + (j & 3);
            const float l = (has_L && v < a.V) ? lrow[b][v] : 0.f;
            z[j] = v < a.V ? l + acc[b][j] : neg_inf();
          }
        }
        const int p = pw + 32 * b + col;
        if (!STAGED && a.z_out != nullptr && p < a.P) {
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int v = vb + 8 * (j >> 2) + (j & 3);
            if (v < a.V) a.z_out[(int64_t)p * a.V + v] = z[j];
          }
        }
        // log-sum-exp in log2 units with the fixed shift cm2: no running
        // maximum.  An element at or above the threshold contributes at
        // least 2^(thr*log2e - cm2) = 2 hb to the group's sum, so a group
        // whose sum stays below hb holds no candidate (the test can only
        // err towards the rare path).
        float sg4[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float e0 = __builtin_amdgcn_exp2f(fmaf(z[4 * g], kLog2e, -cm2[b]));
          const float e1 = __builtin_amdgcn_exp2f(fmaf(z[4 * g + 1], kLog2e, -cm2[b]));
          const float e2 = __builtin_amdgcn_exp2f(fmaf(z[4 * g + 2], kLog2e, -cm2[b]));
          const float e3 = __builtin_amdgcn_exp2f(fmaf(z[4 * g + 3], kLog2e, -cm2[b]));
          sg4[g] = (e0 + e1) + (e2 + e3);
        }
        const float sg = (sg4[0] + sg4[1]) + (sg4[2] + sg4[3]);
        const bool hit = !(sg < hb[b]);
        if (!hit) ss[b] += sg;
        // rare path: some element may enter this lane's top-k, or the sum
        // needs another shift.  A rolled loop that shifts z keeps the code
        // small; z is dead afterwards.  The loop ends after the last element
        // at or above the threshold (which only rises as the list fills).
        if (__any(hit)) {
          if (hit) {
            float m = z[0];
#pragma unroll
            for (int j = 1; j < 16; ++j) m = fmaxf(m, z[j]);
            float s16 = sg;
            if (m == neg_inf()) {
              // nothing to add (under a shift of -inf the sum is NaN)
              s16 = 0.f;
            } else if (!(fmaf(m, kLog2e, -cm2[b]) <= 64.f)) {
              // far above the shift (or the first finite group of a parent
              // without a threshold): shift to this group's maximum
              const float cn = m * kLog2e;
              ss[b] = ss[b] == 0.f ? 0.f
                                   : ss[b] * __builtin_amdgcn_exp2f(cm2[b] - cn);
              cm2[b] = cn;
              s16 = 0.f;
#pragma unroll
              for (int j = 0; j < 16; ++j)
                s16 += __builtin_amdgcn_exp2f(fmaf(z[j], kLog2e, -cn));
            }
            ss[b] += s16;
            const int li = (wave * 64 + lane) * NB + b;
            ZV* lst = lists + li * a.k;
            int cnt = lcount[li];
            int v = vb;
            int jend = 0;
#pragma unroll
            for (int i = 0; i < 16; ++i) jend = z[i] >= thr[b] ? i + 1 : jend;
#pragma unroll 1
            for (int j = 0; j < jend; ++j) {
              const float zj = z[0];
#pragma unroll
              for (int i = 0; i < 15; ++i) z[i] = z[i + 1];
              if (zj >= thr[b] && v < a.V)
                list_insert(lst, a.k, cnt, thr[b], zj, v);
              v += ((j & 3) == 3) ? 5 : 1;
            }
            lcount[li] = cnt;
            hb[b] = __builtin_amdgcn_exp2f(fmaf(thr[b], kLog2e, -cm2[b]) - 1.f);
          }
        }
      }
    }
  };

  // Two waves share each SIMD (waves w and w + NW/2).  The second half of
  // the workgroup runs half a tile behind: while an early wave issues the
  // MFMA chain of a half-tile, its SIMD partner runs the VALU epilogue of
  // the previous one, so the matrix core and the VALU work at the same time
  // instead of both waves contracting, then both exponentiating.  Per tile t:
  //   early: mma(t,0) | epi(t,0) mma(t,1) epi(t,1)
  //   late:  epi(t-1,1) | mma(t,0) epi(t,0) mma(t,1)
  // The barrier at "|" follows the late waves' last read of tile t-1's L
  // rows, so the loads of tile t+1 into that buffer are issued there; the
  // barrier at the end of the tile waits for them.  Tile i of the workgroup
  // is tile id t (its predecessor tp, its successor tn).  During it one
  // thread publishes the id of tile i + 2 at the end; with a queue it takes
  // that tile's ticket just before the tile's loads, so the wait for those
  // loads at the end of the tile also covers the atomic.
  const bool late = NW >= 2 && wave >= NW / 2;
  // a wave with no parents only loads its share of the tiles
  const bool active = pw < a.P;
  const bool taker = tid == (NW >= 2 ? NW / 2 : 0) * 64;
  auto take = [&](int which) __attribute__((always_inline)) {
    // the counter's address as a per-lane value: a uniform address would
    // let the compiler turn the atomic into a wave-wide one that it waits
    // for at once
    int off = which;
    asm volatile("" : "+v"(off));
    return __hip_atomic_fetch_add(tq + off, 1, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
  };
  auto tile = [&](int i, int t, int tp, int tn, const uint4* wt,
                  const float4* lt, uint4* wn, float4* ln,
                  const float4* lp) __attribute__((always_inline)) {
    if (active) {
      if (!late) mma(wt, 0);
      else if (i > 0) epi(tp, 1, lp);
    }
    __syncthreads();
    int ticket = 0;
    if (taker && queued) ticket = take(0);
    if (tn < a.n_tiles) issue(tn, wn, ln);
    if (!active) {
    } else if (!late) {
      epi(t, 0, lt);
      mma(wt, 1);
      epi(t, 1, lt);
    } else {
      mma(wt, 0);
      epi(t, 0, lt);
      mma(wt, 1);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    // (a ticket can only be negative if the queue was not cleared: then the
    // workgroup stops rather than read outside W)
    if (taker && queued)
      sq[(i + 2) & 3] = ticket >= 0 ? 2 * nwg + ticket : a.n_tiles;
    __syncthreads();
  };
  int cur = fixed_id(0);
  if (tid == 0 && queued) sq[1] = fixed_id(1);
  if (cur < a.n_tiles) issue(cur, w0, l0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  // the fragments pass through an opaque statement here, so the compiler
  // neither predicates their loads on the zeroing below nor waits for them
  // before the tile loads above are issued
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const bool past = pw + 32 * b + col >= a.P;
#pragma unroll
    for (int kk = 0; kk < R16; ++kk) {
      uint4 v = __builtin_bit_cast(uint4, uf[b][kk]);
      asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
      if (past) v = make_uint4(0, 0, 0, 0);
      uf[b][kk] = __builtin_bit_cast(bf16x8, v);
    }
  }
  __syncthreads();
  int i = 0, prv = 0;
  // the id of tile i + 1: from the ring with a queue, else computed
  auto next_id = [&](int i) __attribute__((always_inline)) {
    return queued ? __builtin_amdgcn_readfirstlane(sq[(i + 1) & 3])
                  : fixed_id(i + 1);
  };
  while (cur < a.n_tiles) {
    int nxt = next_id(i);
    tile(i, cur, prv, nxt, w0, l0, w1, l1, l1);
    prv = cur;
    cur = nxt;
    ++i;
    if (cur >= a.n_tiles) break;
    nxt = next_id(i);
    tile(i, cur, prv, nxt, w1, l1, w0, l0, l0);
    prv = cur;
    cur = nxt;
    ++i;
  }
  // every ticket of this workgroup has returned: count the workgroup as
  // finished (the answer is looked at after the flush)
  int done = 0;
  if (taker && queued) done = take(1);
  if (active && late && i > 0) epi(prv, 1, ((i - 1) & 1) ? l1 : l0);

#pragma unroll
  for (int b = 0; b < NB; ++b) {
    float c2 = ss[b] > 0.f ? cm2[b] : neg_inf(), s = ss[b];
    combine_halves(c2, s, lane);
    const int p = pw + 32 * b + col;
    if (p < a.P) {
      const int li = (wave * 64 + lane) * NB + b;
      flush_lane(a, p, slice, c2, s, lists + li * a.k, lcount[li], h == 0);
    }
  }
  // the last workgroup to finish clears the queue for the next launch
  if (taker && queued && done == nwg - 1) {
    __hip_atomic_store(&tq[0], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&tq[1], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Thin form for frontiers of at most 32 parents (one parent block), where
// the tiled kernel has a single wave with parents and the launch is bound by
// streaming W one tile ahead.  Every wave of the workgroup takes its own
// 32-row pieces of the slice (pieces wave, wave + 8, ...), loads their W
// rows from global memory straight into MFMA operand registers (no LDS
// staging, no barrier in the loop), and runs the same epilogue on its 16
// rows per lane; the waves' (max, sum) partials meet in LDS at the end, and
// every lane flushes its own top-k list.
constexpr int kThinWaves = 8;

template <int R16>
__global__ __launch_bounds__(kThinWaves * 64) void markov_topk_thin(
    K1Args a) {
  constexpr int CH = 2 * R16;  // 16-byte chunks per W row
  extern __shared__ __align__(16) unsigned char smem[];
  ZV* lists = reinterpret_cast<ZV*>(smem);
  __shared__ float2 wpart[kThinWaves][32];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, col = lane & 31;
  const int slice = blockIdx.x;
  const int r0 = slice * a.vslice, r1 = min(r0 + a.vslice, a.V);
  const bool has_L = a.L != nullptr;
  const int p = col;
  const bool valid = p < a.P;
  const int pc = valid ? p : a.P - 1;
  float thr = valid ? (a.theta ? a.theta[p] : neg_inf()) : pos_inf();
  int64_t row = a.plrow ? a.plrow[pc]
                        : (int64_t)(a.group_fp > 0 ? pc / a.group_fp : pc) *
                                  a.lrow_mul +
                              a.lrow_add;
  row = row < 0 ? 0 : (row >= a.L_rows ? a.L_rows - 1 : row);
  const float* lrow = has_L ? a.L + row * a.lstride : nullptr;
  bf16x8 uf[R16];
  // Rank step kk of lane half h takes the rank chunk R16*h + kk (a
  // relabelling of the contraction index, the same for U and W), so that a
  // lane's W loads walk a contiguous half row.
  if (a.upack != nullptr) {
    // block 0; chunk c of the packed rows sits at (c/2)*64 + (c%2)*32 + col
#pragma unroll
    for (int kk = 0; kk < R16; ++kk) {
      const int c = R16 * h + kk;
      uf[kk] = __builtin_bit_cast(bf16x8,
                                  a.upack[(c >> 1) * 64 + (c & 1) * 32 + col]);
    }
  } else {
    const int ptk = min(max(a.ptok[pc], 0), a.V - 1);
    const uint4* up =
        reinterpret_cast<const uint4*>(a.U) + (int64_t)ptk * CH + R16 * h;
#pragma unroll
    for (int kk = 0; kk < R16; ++kk)
      uf[kk] = __builtin_bit_cast(bf16x8, up[kk]);
  }
  if (!valid) {
#pragma unroll
    for (int kk = 0; kk < R16; ++kk)
      uf[kk] = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
  }
  ZV* lst = lists + (wave * 64 + lane) * a.k;
  int cnt = 0;
  float cm2 = neg_inf(), ss = 0.f;
  const uint4* Wg = reinterpret_cast<const uint4*>(a.W);
  for (int v0 = r0 + 32 * wave; v0 < r1; v0 += 32 * kThinWaves) {
    // W rows v0 + col (rows past V read row V - 1; their outputs are
    // masked), chunks R16*h + kk: the MFMA operand of rank step kk
    const uint4* wp = Wg + (int64_t)min(v0 + col, a.V - 1) * CH + R16 * h;
    bf16x8 wf[R16];
#pragma unroll
    for (int kk = 0; kk < R16; ++kk)
      wf[kk] = __builtin_bit_cast(bf16x8, wp[kk]);
    // register j of this lane holds vocab vb + 8*(j/4) + j%4
    const int vb = v0 + 4 * h;
    const bool full = v0 + 32 <= a.V;
    float4 lq[4];
    if (has_L && full && a.vec_ok) {
      // non-temporal: read once, while W is read again by the next depth
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 y = __builtin_nontemporal_load(
            reinterpret_cast<const f32x4*>(lrow + vb + 8 * g));
        lq[g] = make_float4(y.x, y.y, y.z, y.w);
      }
    }
    f32x16 acc;
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = 0.f;
#pragma unroll
    for (int kk = 0; kk < R16; ++kk)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[kk], uf[kk], acc, 0,
                                                    0, 0);
    float z[16];
    if (full && a.vec_ok) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 l4 = has_L ? lq[g] : make_float4(0.f, 0.f, 0.f, 0.f);
        z[4 * g + 0] = l4.x + acc[4 * g + 0];
        z[4 * g + 1] = l4.y + acc[4 * g + 1];
        z[4 * g + 2] = l4.z + acc[4 * g + 2];
        z[4 * g + 3] = l4.w + acc[4 * g + 3];
      }
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int v = vb + 8 * (j >> 2) + (j & 3);
        const float l = (has_L && v < a.V) ? lrow[v] : 0.f;
        z[j] = v < a.V ? l + acc[j] : neg_inf();
      }
    }
    float m = z[0];
#pragma unroll
    for (int j = 1; j < 16; ++j) m = fmaxf(m, z[j]);
    if (a.z_out != nullptr && valid) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int v = vb + 8 * (j >> 2) + (j & 3);
        if (v < a.V) a.z_out[(int64_t)p * a.V + v] = z[j];
      }
    }
    // online log-sum-exp in log2 units
    const float m2 = m * kLog2e;
    if (m2 > cm2) {
      ss *= __builtin_amdgcn_exp2f(cm2 - m2);
      cm2 = m2;
    }
    if (m != neg_inf()) {
      float sg[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float e0 = __builtin_amdgcn_exp2f(fmaf(z[4 * g], kLog2e, -cm2));
        const float e1 = __builtin_amdgcn_exp2f(fmaf(z[4 * g + 1], kLog2e, -cm2));
        const float e2 = __builtin_amdgcn_exp2f(fmaf(z[4 * g + 2], kLog2e, -cm2));
        const float e3 = __builtin_amdgcn_exp2f(fmaf(z[4 * g + 3], kLog2e, -cm2));
        sg[g] = (e0 + e1) + (e2 + e3);
      }
      ss += (sg[0] + sg[1]) + (sg[2] + sg[3]);
    }
    // rare path, in vocabulary order (the list's tie rule needs it)
    if (m >= thr) {
      int v = vb;
      int jend = 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) jend = z[i] >= thr ? i + 1 : jend;
#pragma unroll 1
      for (int j = 0; j < jend; ++j) {
        const float zj = z[0];
#pragma unroll
        for (int i = 0; i < 15; ++i) z[i] = z[i + 1];
        if (zj >= thr && v < a.V) list_insert(lst, a.k, cnt, thr, zj, v);
        v += ((j & 3) == 3) ? 5 : 1;
      }
    }
  }
  // partials: the two halves of the wave, then the waves
  combine_halves(cm2, ss, lane);
  if (h == 0) wpart[wave][col] = make_float2(cm2, ss);
  __syncthreads();
  if (wave == 0 && h == 0 && valid) {
    float c = neg_inf();
#pragma unroll
    for (int w = 0; w < kThinWaves; ++w) c = fmaxf(c, wpart[w][col].x);
    float s = 0.f;
    if (c != neg_inf()) {
#pragma unroll
      for (int w = 0; w < kThinWaves; ++w) {
        const float2 e = wpart[w][col];
        if (e.x != neg_inf()) s += e.y * __builtin_amdgcn_exp2f(e.x - c);
      }
    }
    a.part_c[(int64_t)slice * a.P + p] = c;
    a.part_s[(int64_t)slice * a.P + p] = s;
  }
  if (valid && cnt > 0) {
    const int pos = atomicAdd(&a.gcnt[p], cnt);
    float* gz = a.gz + (int64_t)p * a.cap + pos;
    int32_t* gv = a.gv + (int64_t)p * a.cap + pos;
    for (int i = 0; i < cnt; ++i) {
      gz[i] = lst[i].z;
      gv[i] = lst[i].v;
    }
  }
}

template <int R16>
hipError_t go_thin(const K1Plan& pl, const K1Args& a, hipStream_t s) {
  auto fn = markov_topk_thin<R16>;
  hipError_t e = allow_lds(reinterpret_cast<const void*>(fn), pl.lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fn, pl.grid, pl.block, pl.lds, s, a);
  return hipGetLastError();
}

template <int NB, int NW, int R16, bool STAGED, int LSL = kLdsRowSlots>
hipError_t go_mfma(const K1Plan& pl, const K1Args& a, hipStream_t s) {
  auto fn = markov_topk_mfma<NB, NW, R16, STAGED, LSL>;
  hipError_t e = allow_lds(reinterpret_cast<const void*>(fn), pl.lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fn, pl.grid, pl.block, pl.lds, s, a);
  return hipGetLastError();
}

// Launcher for one rank (r = 16*R16) and row mode: picks the (NB, NW)
// instantiation.
template <int R16, bool STAGED>
hipError_t launch_mfma_rank(const K1Plan& pl, const K1Args& a,
                            hipStream_t s) {
  if constexpr (!STAGED) {
    if (pl.thin) return go_thin<R16>(pl, a, s);
  }
  if (pl.NB == 1) {
    if (pl.NW != 8) return go_mfma<1, 1, R16, STAGED>(pl, a, s);
    // long lists leave room for fewer staged L rows
    if constexpr (STAGED) {
      if (pl.lslots == kSmallRowSlots)
        return go_mfma<1, 8, R16, STAGED, kSmallRowSlots>(pl, a, s);
    }
    return go_mfma<1, 8, R16, STAGED>(pl, a, s);
  }
  switch (pl.NW) {
    case 8: return go_mfma<2, 8, R16, STAGED>(pl, a, s);
    case 4: return go_mfma<2, 4, R16, STAGED>(pl, a, s);
    case 2: return go_mfma<2, 2, R16, STAGED>(pl, a, s);
    default: return go_mfma<2, 1, R16, STAGED>(pl, a, s);
  }
}

}  // namespace pct
