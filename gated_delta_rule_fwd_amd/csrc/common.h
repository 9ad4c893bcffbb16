// Device helpers shared by the gfx950 kernels of the gated delta-rule library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace kda {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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

// x + x of lane ^ 16, and x + x of lane ^ 32 (gfx950 lane-swap moves)
__device__ __forceinline__ float xor16_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum over aligned groups of W consecutive lanes with DPP lane moves within
// rows of 16 and lane-swap moves across them (no LDS traffic), the result in
// every lane of the group.  W = 4, 8, 16, 32 or 64.
template <int W>
__device__ __forceinline__ float dpp_group_sum(float x) {
  auto mov = [](float v, auto ctrl) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), decltype(ctrl)::value,
                                                      0xf, 0xf, false));
  };
  using xor1 = std::integral_constant<int, 0xB1>;   // quad_perm [1,0,3,2]
  using xor2 = std::integral_constant<int, 0x4E>;   // quad_perm [2,3,0,1]
  using hmir = std::integral_constant<int, 0x141>;  // row_half_mirror (within 8)
  using ror4 = std::integral_constant<int, 0x124>;  // row_ror:4 (within 16)
  using ror8 = std::integral_constant<int, 0x128>;  // row_ror:8 (within 16)
  if constexpr (W == 8) x += mov(x, hmir{});
  if constexpr (W >= 16) {
    x += mov(x, ror8{});
    x += mov(x, ror4{});
  }
  x += mov(x, xor2{});
  x += mov(x, xor1{});
  if constexpr (W >= 32) x = xor16_sum(x);
  if constexpr (W >= 64) x = xor32_sum(x);
  return x;
}

// Optional input transforms (TileOPs "Linear Attention Operators", GDNFwdOp
// and KDAFwdOp parameter lists).  With a raw gate the log-space decay is
// -exp(A_log) * softplus(gate + dt_bias) (ejkernel kda_decay, the Mamba-style
// discretisation), floored at `lower`; with raw beta the update strength is
// sigmoid(beta), or twice it when negative eigenvalues are allowed.
struct Transforms {
  const float* A_log;     // [H]; non-NULL: the decay input holds the raw gate
  const float* dt_bias;   // [H] (per-head gate) or [H, DK] (per-channel); NULL = 0
  float lower;            // log-space floor of the decay (-inf: none)
  int beta_mode;          // 0 beta as given, 1 sigmoid, 2 twice the sigmoid
};

// softplus(x) = log(1 + e^x) = max(x, 0) + log(1 + e^-|x|): no overflow, and an
// absolute error of a few fp32 ulps of 1 (what the decay sums need).
__device__ __forceinline__ float softplus_f(float x) {
  return fmaxf(x, 0.f) + __logf(1.f + __expf(-fabsf(x)));
}
// negA = -exp(A_log[h]) of the head
__device__ __forceinline__ float gate_decay(float gate, float negA, float bias, float lower) {
  return fmaxf(negA * softplus_f(gate + bias), lower);
}
__device__ __forceinline__ float beta_transform(float b, int mode) {
  if (mode == 0) return b;
  const float s = 1.f / (1.f + __expf(-b));
  return mode == 2 ? 2.f * s : s;
}

// Sum over the lanes that share lane % W (W = 8 or 16): within each 16-lane
// row with DPP rotations, then across rows with the lane-swap moves.
template <int W>
__device__ __forceinline__ float rowgroup_sum(float x) {
  auto ror = [](float v, auto ctrl) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), decltype(ctrl)::value,
                                                      0xf, 0xf, false));
  };
  if constexpr (W == 8) x += ror(x, std::integral_constant<int, 0x128>{});   // row_ror:8
  return xor32_sum(xor16_sum(x));
}

// Inclusive prefix sum over the 64 lanes of a wave, with its exclusive
// counterpart (lane i: the inclusive sum of lane i - 1, 0 in lane 0) and the
// wave's total, all without LDS traffic: DPP right shifts within each row of
// 16 lanes (a lane with no source adds 0), then the totals of the earlier
// rows, read from lanes 15, 31 and 47.
struct WaveScan { float incl, excl, total; };
__device__ __forceinline__ WaveScan wave_scan(float x) {
  auto shr = [](float v, auto ctrl) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), decltype(ctrl)::value,
                                                      0xf, 0xf, false));
  };
  auto lane_val = [](float v, int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l)); };
  x += shr(x, std::integral_constant<int, 0x111>{});   // row_shr:1
  x += shr(x, std::integral_constant<int, 0x112>{});   // row_shr:2
  x += shr(x, std::integral_constant<int, 0x114>{});   // row_shr:4
  x += shr(x, std::integral_constant<int, 0x118>{});   // row_shr:8
  const int lane = __lane_id(), row = lane >> 4;
  const float r0 = lane_val(x, 15), r1 = lane_val(x, 31), r2 = lane_val(x, 47);
  const float before = row == 0 ? 0.f : row == 1 ? r0 : row == 2 ? r0 + r1 : (r0 + r1) + r2;
  x += before;
  WaveScan w;
  w.incl = x;
  const float prev = shr(x, std::integral_constant<int, 0x111>{});
  const float e0 = lane_val(x, 15), e1 = lane_val(x, 31), e2 = lane_val(x, 47);
  const float edge = row == 0 ? 0.f : row == 1 ? e0 : row == 2 ? e1 : e2;
  w.excl = (lane & 15) == 0 ? edge : prev;
  w.total = lane_val(x, 63);
  return w;
}

__device__ __forceinline__ float inv_norm(float sumsq) {
  // 1 / max(||x||_2, 1e-12): the hardware reciprocal square root (about
  // 1 ulp), capped where the norm is below 1e-12 (a NaN sum gives the cap)
  return fminf(__builtin_amdgcn_rsqf(sumsq), 1e12f);
}

}  // namespace kda
