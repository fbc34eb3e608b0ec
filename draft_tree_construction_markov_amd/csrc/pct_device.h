// pct_device.h -- device-side helpers shared by the libpctree kernels
// (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pct {

constexpr float kLog2e = 1.4426950408889634f;
constexpr double kLn2 = 0.6931471805599453094;
constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }
__device__ __forceinline__ float pos_inf() { return __builtin_inff(); }

// ---------------------------------------------------------------------
// Order-preserving map of fp32 onto uint32 (ascending float -> ascending
// integer); the keys below use it inverted so that ascending keys mean
// descending scores.
__device__ __forceinline__ uint32_t float_to_ordered(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float ordered_to_float(uint32_t o) {
  uint32_t u = (o & 0x80000000u) ? (o & 0x7fffffffu) : ~o;
  return __uint_as_float(u);
}

// Tree key: ascending order = (score desc, parent pool id asc, token asc).
// Bits: [63:32] inverted ordered score, [31:18] parent pool id + 1 (the root
// is -1 -> 0), [17:0] token.
constexpr int kTokBits = 18;
constexpr int kPidBits = 14;
__device__ __forceinline__ uint64_t make_key(float s, int32_t ppid,
                                             int32_t tok) {
  uint64_t hi = (uint64_t)(~float_to_ordered(s));
  return (hi << 32) | ((uint64_t)(uint32_t)(ppid + 1) << kTokBits) |
         (uint64_t)(uint32_t)tok;
}
__device__ __forceinline__ float key_score(uint64_t key) {
  return ordered_to_float(~(uint32_t)(key >> 32));
}
__device__ __forceinline__ int32_t key_ppid(uint64_t key) {
  return (int32_t)((key >> kTokBits) & ((1u << kPidBits) - 1)) - 1;
}
__device__ __forceinline__ int32_t key_tok(uint64_t key) {
  return (int32_t)(key & ((1u << kTokBits) - 1));
}

// (z desc, token asc): true if (za, va) comes before (zb, vb)
__device__ __forceinline__ bool zv_before(float za, int32_t va, float zb,
                                          int32_t vb) {
  return za > zb || (za == zb && va < vb);
}

// ---------------------------------------------------------------------
// Wave-wide all-reductions (64 lanes) on DPP: within each row of 16 lanes a
// quad xor-1 / xor-2 exchange and row rotations by 4 and 8 give every lane
// its row's result; the four row results are then read with readlane, so
// the result is the same on every lane.  (Cross-lane shuffles through
// ds_bpermute have a long latency; these are VALU modifiers.)
template <int CTRL>
__device__ __forceinline__ int dpp_i(int x) {
  return __builtin_amdgcn_mov_dpp(x, CTRL, 0xf, 0xf, false);
}
constexpr int kDppXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kDppRor4 = 0x124; // row_ror:4
constexpr int kDppRor8 = 0x128; // row_ror:8

template <typename T>
struct Bits32 {
  static __device__ __forceinline__ int to(T x) {
    return __builtin_bit_cast(int, x);
  }
  static __device__ __forceinline__ T from(int x) {
    return __builtin_bit_cast(T, x);
  }
};

template <typename T, typename Op>
__device__ __forceinline__ T wave_allreduce32(T x, Op op) {
  x = op(x, Bits32<T>::from(dpp_i<kDppXor1>(Bits32<T>::to(x))));
  x = op(x, Bits32<T>::from(dpp_i<kDppXor2>(Bits32<T>::to(x))));
  x = op(x, Bits32<T>::from(dpp_i<kDppRor4>(Bits32<T>::to(x))));
  x = op(x, Bits32<T>::from(dpp_i<kDppRor8>(Bits32<T>::to(x))));
  const int b = Bits32<T>::to(x);
  const T r0 = Bits32<T>::from(__builtin_amdgcn_readlane(b, 0));
  const T r1 = Bits32<T>::from(__builtin_amdgcn_readlane(b, 16));
  const T r2 = Bits32<T>::from(__builtin_amdgcn_readlane(b, 32));
  const T r3 = Bits32<T>::from(__builtin_amdgcn_readlane(b, 48));
  return op(op(r0, r1), op(r2, r3));
}

template <int CTRL>
__device__ __forceinline__ double dpp_d(double x) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const int lo = dpp_i<CTRL>((int)(uint32_t)u);
  const int hi = dpp_i<CTRL>((int)(uint32_t)(u >> 32));
  return __builtin_bit_cast(double,
                            ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}
__device__ __forceinline__ double readlane_d(double x, int l) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)u, l);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
template <typename Op>
__device__ __forceinline__ double wave_allreduce_d(double x, Op op) {
  x = op(x, dpp_d<kDppXor1>(x));
  x = op(x, dpp_d<kDppXor2>(x));
  x = op(x, dpp_d<kDppRor4>(x));
  x = op(x, dpp_d<kDppRor8>(x));
  return op(op(readlane_d(x, 0), readlane_d(x, 16)),
            op(readlane_d(x, 32), readlane_d(x, 48)));
}

__device__ __forceinline__ float wave_max(float x) {
  return wave_allreduce32(x, [](float a, float b) { return fmaxf(a, b); });
}
__device__ __forceinline__ int wave_max(int x) {
  return wave_allreduce32(x, [](int a, int b) { return a > b ? a : b; });
}
__device__ __forceinline__ int wave_sum(int x) {
  return wave_allreduce32(x, [](int a, int b) { return a + b; });
}
__device__ __forceinline__ float wave_sum(float x) {
  return wave_allreduce32(x, [](float a, float b) { return a + b; });
}
__device__ __forceinline__ double wave_sum(double x) {
  return wave_allreduce_d(x, [](double a, double b) { return a + b; });
}
__device__ __forceinline__ double wave_max(double x) {
  return wave_allreduce_d(x, [](double a, double b) { return a > b ? a : b; });
}

// best (z desc, v asc) pair over the wave, result on every lane
__device__ __forceinline__ void wave_best_zv(float& z, int32_t& v) {
  auto step = [&](float z2, int32_t v2) {
    if (zv_before(z2, v2, z, v)) {
      z = z2;
      v = v2;
    }
  };
  step(Bits32<float>::from(dpp_i<kDppXor1>(Bits32<float>::to(z))),
       dpp_i<kDppXor1>(v));
  step(Bits32<float>::from(dpp_i<kDppXor2>(Bits32<float>::to(z))),
       dpp_i<kDppXor2>(v));
  step(Bits32<float>::from(dpp_i<kDppRor4>(Bits32<float>::to(z))),
       dpp_i<kDppRor4>(v));
  step(Bits32<float>::from(dpp_i<kDppRor8>(Bits32<float>::to(z))),
       dpp_i<kDppRor8>(v));
  const int zb = Bits32<float>::to(z);
  float bz = Bits32<float>::from(__builtin_amdgcn_readlane(zb, 0));
  int32_t bv = __builtin_amdgcn_readlane(v, 0);
#pragma unroll
  for (int r = 1; r < 4; ++r) {
    const float z2 = Bits32<float>::from(__builtin_amdgcn_readlane(zb, 16 * r));
    const int32_t v2 = __builtin_amdgcn_readlane(v, 16 * r);
    if (zv_before(z2, v2, bz, bv)) {
      bz = z2;
      bv = v2;
    }
  }
  z = bz;
  v = bv;
}

// The value held by lane (lane ^ 32), via the gfx950 permlane32 swap.
__device__ __forceinline__ float swap_halves(float x, int lane) {
  const int b = Bits32<float>::to(x);
  const auto pr = __builtin_amdgcn_permlane32_swap(b, b, false, false);
  return Bits32<float>::from(lane < 32 ? pr[1] : pr[0]);
}

__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

}  // namespace pct
