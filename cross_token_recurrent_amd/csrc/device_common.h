// Device-side helpers shared by the RLT HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rlt {

// bf16 values are stored as raw 16-bit patterns.
typedef uint16_t bf16_t;

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round-to-nearest-even fp32 -> bf16 (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f));
}

// Two values packed low | high << 16, both rounded to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __attribute__((ext_vector_type(2))) float f32x2_v;
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_v;
  const f32x2_v x = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2_v));
}

// Value after a round trip through the storage type (identity for fp32).
template <typename T> __device__ __forceinline__ float round_to(float x);
template <> __device__ __forceinline__ float round_to<float>(float x) { return x; }
template <> __device__ __forceinline__ float round_to<bf16_t>(float x) { return bf16_to_f32(f32_to_bf16(x)); }

template <typename T> __device__ __forceinline__ float load_as_f32(const T* p);
template <> __device__ __forceinline__ float load_as_f32<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float load_as_f32<bf16_t>(const bf16_t* p) { return bf16_to_f32(*p); }

template <typename T> __device__ __forceinline__ void store_from_f32(T* p, float v);
template <> __device__ __forceinline__ void store_from_f32<float>(float* p, float v) { *p = v; }
template <> __device__ __forceinline__ void store_from_f32<bf16_t>(bf16_t* p, float v) { *p = f32_to_bf16(v); }

// Load 8 consecutive elements (16-byte aligned for bf16, 32-byte for fp32) as fp32.
__device__ __forceinline__ void load8(const bf16_t* p, float (&v)[8]) {
  const uint4 q = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8(const float* p, float (&v)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// Load 4 consecutive elements (8-byte aligned for bf16, 16-byte for fp32) as fp32.
__device__ __forceinline__ void load4(const bf16_t* p, float (&v)[4]) {
  const uint2 q = *reinterpret_cast<const uint2*>(p);
  v[0] = __uint_as_float(q.x << 16);
  v[1] = __uint_as_float(q.x & 0xffff0000u);
  v[2] = __uint_as_float(q.y << 16);
  v[3] = __uint_as_float(q.y & 0xffff0000u);
}
__device__ __forceinline__ void load4(const float* p, float (&v)[4]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
}

__device__ __forceinline__ float gelu_erf(float x) { return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f)); }
__device__ __forceinline__ float silu_f(float x) { return x / (1.0f + expf(-x)); }
__device__ __forceinline__ float sigmoid_f(float x) { return 1.0f / (1.0f + expf(-x)); }

// Cross-lane data movement inside a row of 16 lanes (DPP, no LDS round trip).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;          // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;          // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;   // lane i <-> 7-i within 8
constexpr int kDppMirror = 0x140;       // lane i <-> 15-i within 16

// All-reduce over aligned groups of WIDTH lanes (all lanes of a group must be active).
// Groups up to 16 use DPP butterflies; 64 adds the four row results read back with
// v_readlane in a fixed order, so every lane (and every wave) gets bit-identical results.
template <int WIDTH>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(WIDTH == 1 || WIDTH == 2 || WIDTH == 4 || WIDTH == 8 || WIDTH == 16 || WIDTH == 32 || WIDTH == 64,
                "group width");
  if constexpr (WIDTH >= 2) v += dpp_mov<kDppXor1>(v);
  if constexpr (WIDTH >= 4) v += dpp_mov<kDppXor2>(v);
  if constexpr (WIDTH >= 8) v += dpp_mov<kDppHalfMirror>(v);
  if constexpr (WIDTH >= 16) v += dpp_mov<kDppMirror>(v);
  if constexpr (WIDTH == 32) v += __shfl_xor(v, 16, 64);
  if constexpr (WIDTH == 64) {
    const float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    const float b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
    const float c = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    const float d = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
    v = (a + b) + (c + d);
  }
  return v;
}
template <int WIDTH>
__device__ __forceinline__ float group_max(float v) {
  static_assert(WIDTH == 1 || WIDTH == 2 || WIDTH == 4 || WIDTH == 8 || WIDTH == 16 || WIDTH == 32 || WIDTH == 64,
                "group width");
  if constexpr (WIDTH >= 2) v = fmaxf(v, dpp_mov<kDppXor1>(v));
  if constexpr (WIDTH >= 4) v = fmaxf(v, dpp_mov<kDppXor2>(v));
  if constexpr (WIDTH >= 8) v = fmaxf(v, dpp_mov<kDppHalfMirror>(v));
  if constexpr (WIDTH >= 16) v = fmaxf(v, dpp_mov<kDppMirror>(v));
  if constexpr (WIDTH == 32) v = fmaxf(v, __shfl_xor(v, 16, 64));
  if constexpr (WIDTH == 64) {
    const float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    const float b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
    const float c = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    const float d = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
    v = fmaxf(fmaxf(a, b), fmaxf(c, d));
  }
  return v;
}

}  // namespace rlt
