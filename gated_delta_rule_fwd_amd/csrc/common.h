// Device helpers shared by the gfx950 kernels of the gated delta-rule library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

enum { DECAY_NONE = 0, DECAY_HEAD = 1, DECAY_CHANNEL = 2 };

// Activation element types: raw fp32, or bf16 carried as its 16-bit pattern.
struct bf16_t { uint16_t bits; };

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even fp32 -> bf16 bit pattern (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

template <typename In> struct act;
template <> struct act<float> {
  static constexpr int kVec = 4;  // elements per 16-byte load
  __device__ static float load1(const float* p) { return *p; }
  __device__ static float cvt(float x) { return x; }
  __device__ static void load_vec(const float* p, float (&out)[4]) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(p);
    out[0] = v[0]; out[1] = v[1]; out[2] = v[2]; out[3] = v[3];
  }
};
template <> struct act<bf16_t> {
  static constexpr int kVec = 8;
  __device__ static float load1(const bf16_t* p) { return bf16_to_f32(p->bits); }
  __device__ static float cvt(bf16_t x) { return bf16_to_f32(x.bits); }
  __device__ static void load_vec(const bf16_t* p, float (&out)[8]) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(w[i] << 16);
      out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};

// Butterfly sum over groups of `width` consecutive lanes (width a power of 2 <= 64).
template <int width>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int off = width / 2; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

__device__ __forceinline__ float inv_norm(float sumsq) {
  // 1 / max(||x||_2, 1e-12)
  return 1.0f / fmaxf(sqrtf(sumsq), 1e-12f);
}

}  // namespace kda
