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
// wave reductions (64 lanes)
template <typename T>
__device__ __forceinline__ T wave_max(T x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    T y = __shfl_xor(x, o, kWave);
    x = y > x ? y : x;
  }
  return x;
}
template <typename T>
__device__ __forceinline__ T wave_min(T x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    T y = __shfl_xor(x, o, kWave);
    x = y < x ? y : x;
  }
  return x;
}
template <typename T>
__device__ __forceinline__ T wave_sum(T x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, kWave);
  return x;
}
// best (z desc, v asc) pair over the wave, result on every lane
__device__ __forceinline__ void wave_best_zv(float& z, int32_t& v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    float z2 = __shfl_xor(z, o, kWave);
    int32_t v2 = __shfl_xor(v, o, kWave);
    if (zv_before(z2, v2, z, v)) {
      z = z2;
      v = v2;
    }
  }
}

__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

}  // namespace pct
