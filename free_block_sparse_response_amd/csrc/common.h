// Internal device helpers shared by the SparsePR kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace spr {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kMaxGroups = 1024;

// ---------------------------------------------------------------------------------
// SplitMix64 mixer (Steele, Lea, Flood, OOPSLA 2014): first output of a generator whose
// state is x. A token's selection rank is h = mix(mix(mix(seed ^ stream) ^ head) ^ i).
// ---------------------------------------------------------------------------------
__host__ __device__ inline uint64_t splitmix64(uint64_t x) {
  uint64_t z = x + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
__device__ inline uint64_t head_hash_base(uint64_t seed, uint64_t stream, uint64_t head) {
  return splitmix64(splitmix64(seed ^ stream) ^ head);
}

enum Stream : uint64_t { kStreamSampled = 1, kStreamKeyInit = 2, kStreamQueryInit = 3, kStreamProbes = 4 };

// ---------------------------------------------------------------------------------
// Element loads/stores for the two storage types.
// ---------------------------------------------------------------------------------
__device__ inline float to_f32(float x) { return x; }
__device__ inline float to_f32(bf16 x) { return (float)x; }
template <typename T> __device__ inline T from_f32(float x);
template <> __device__ inline float from_f32<float>(float x) { return x; }
template <> __device__ inline bf16 from_f32<bf16>(float x) { return (bf16)x; }

// ---------------------------------------------------------------------------------
// Wave helpers.
// ---------------------------------------------------------------------------------
__device__ inline int lane_id() { return threadIdx.x & (kWave - 1); }
__device__ inline uint64_t lanemask_lt() { return (1ull << lane_id()) - 1ull; }

template <typename T> __device__ inline T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ inline int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ inline long long wave_sum_ll(long long v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
// Inclusive prefix sum over the wave (lane order).
__device__ inline int wave_incl_scan(int v) {
  const int l = lane_id();
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    int t = __shfl_up(v, o, kWave);
    if (l >= o) v += t;
  }
  return v;
}
__device__ inline long long wave_incl_scan_ll(long long v) {
  const int l = lane_id();
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    long long t = __shfl_up(v, o, kWave);
    if (l >= o) v += t;
  }
  return v;
}

// Lanes of this wave whose `key` equals mine (only lanes with `valid`); key < 2^bits.
__device__ inline uint64_t wave_match(int key, bool valid, int bits) {
  uint64_t m = __ballot(valid);
  for (int b = 0; b < bits; ++b) {
    uint64_t one = __ballot(valid && ((key >> b) & 1));
    m &= ((key >> b) & 1) ? one : ~one;
  }
  return valid ? m : 0ull;
}

// The same among lanes 0 .. 31 only (a lane >= 32 must pass valid = false): 32-bit masks,
// half the vector work per key bit.
__device__ inline uint32_t wave_match_lo(int key, bool valid, int bits) {
  uint32_t m = (uint32_t)__ballot(valid);
  for (int b = 0; b < bits; ++b) {
    const uint32_t one = (uint32_t)__ballot(valid && ((key >> b) & 1));
    m &= one ^ (uint32_t)(((key >> b) & 1) - 1);  // one if my bit is set, else ~one
  }
  return valid ? m : 0u;
}

__device__ inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Value of lane l ^ 32 (the other half of the wave), by gfx950's v_permlane32_swap (a VALU
// swap of the two 32-lane halves, no LDS round trip).
__device__ inline float xor32(float v) {
  const unsigned u = __float_as_uint(v);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(lane_id() < 32 ? r[1] : r[0]);
}

}  // namespace spr
