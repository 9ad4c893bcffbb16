// Backward of the gated delta rule: the gradients of (o, final state) with
// respect to q, k, v, beta, the decay and the initial state, given do and the
// final-state gradient (TileOPs "Linear Attention Operators",
// DeltaNetChunkBwdOp and GLAChunkBwdOp; kda-neuron-kernels README,
// kda_chunk_step_exact_bwd: dq, dk, dv, dg, dbeta, dstate_in).
//
// The chunked kernels (backward_chunked.hip) produce dv, the initial-state
// gradient, dbeta, the decay's gradient and dq, dk (through the norm and the
// scale, unless value heads share q/k heads: then of the normalised rows,
// added up over the group).  Here: clearing what is added up rather than
// written, the dispatch, and two last elementwise kernels, one carrying
// grouped heads' dq and dk through the L2 norm and the scale, one applying
// the chain rule of the raw-gate and raw-beta transforms.
#include "common.h"
#include "launch.h"

namespace kda {
namespace {

// dq, dk hold the gradients of the normalised (and scaled) rows; carry them
// through x -> scale x / max(||x||, 1e-12), in place.  One wave per row of q
// or k (rows of q first, then of k).
template <int DK, typename In>
__global__ __launch_bounds__(256) void norm_bwd_kernel(const In* __restrict__ q, const In* __restrict__ k,
                                                       float* __restrict__ dq, float* __restrict__ dk,
                                                       long rows, float scale, int l2norm) {
  constexpr int CPL = (DK + 63) / 64;
  const int lane = threadIdx.x & 63;
  const long w = static_cast<long>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (w >= 2 * rows) return;
  const bool isq = w < rows;
  const long row = isq ? w : w - rows;
  const In* x = (isq ? q : k) + row * DK;
  float* g = (isq ? dq : dk) + row * DK;
  const float sc = isq ? scale : 1.f;
  float xv[CPL], gv[CPL], sq = 0.f;
#pragma unroll
  for (int e = 0; e < CPL; ++e) {
    const int c = lane + 64 * e;
    xv[e] = c < DK ? act<In>::load1(x + c) : 0.f;
    gv[e] = c < DK ? g[c] : 0.f;
    sq += xv[e] * xv[e];
  }
  if (!l2norm) {
#pragma unroll
    for (int e = 0; e < CPL; ++e)
      if (lane + 64 * e < DK) g[lane + 64 * e] = sc * gv[e];
    return;
  }
  sq = dpp_group_sum<64>(sq);
  const float n = sqrtf(sq);
  if (n > 1e-12f) {
    const float in = 1.f / n;
    float proj = 0.f;
#pragma unroll
    for (int e = 0; e < CPL; ++e) proj += xv[e] * in * gv[e];
    proj = dpp_group_sum<64>(proj);
#pragma unroll
    for (int e = 0; e < CPL; ++e)
      if (lane + 64 * e < DK) g[lane + 64 * e] = sc * (gv[e] - xv[e] * in * proj) * in;
  } else {
#pragma unroll
    for (int e = 0; e < CPL; ++e)
      if (lane + 64 * e < DK) g[lane + 64 * e] = sc * gv[e] * 1e12f;
  }
}

// The raw-gate / raw-beta chain rule, in place: dbeta and ddecay hold the
// gradients of the transformed beta and decay; they become those of the raw
// inputs, and dA_log / ddt_bias collect their sums (atomic adds).  Where the
// floor is taken the decay is the constant floor and gets no gradient.
// Elements n of [B, T, H] (or [B, T, H, DK] per channel, W = DK).
template <typename In>
__global__ void tf_bwd_kernel(const In* __restrict__ beta, const In* __restrict__ gate,
                              float* __restrict__ dbeta, float* __restrict__ dgate,
                              float* __restrict__ dA_log, float* __restrict__ dbias, Transforms tf,
                              int H, int W, long ntok) {
  const long tot = ntok * W;
  for (long n = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x; n < tot;
       n += static_cast<long>(gridDim.x) * blockDim.x) {
    const long t = n / W;            // token-head index
    const int h = static_cast<int>(t % H), c = static_cast<int>(n % W);
    if (c == 0 && tf.beta_mode) {
      const float sgm = 1.f / (1.f + __expf(-act<In>::load1(beta + t)));
      dbeta[t] *= sgm * (1.f - sgm) * (tf.beta_mode == 2 ? 2.f : 1.f);
    }
    if (tf.A_log && dgate) {
      const float x = act<In>::load1(gate + n) + (tf.dt_bias ? tf.dt_bias[W == 1 ? h : h * W + c] : 0.f);
      const float negA = -__expf(tf.A_log[h]);
      const float raw = negA * softplus_f(x);
      const float gd = dgate[n];
      const bool live = raw >= tf.lower;
      const float dx = live ? gd * negA / (1.f + __expf(-x)) : 0.f;
      dgate[n] = dx;
      if (live) atomicAdd(dA_log + h, gd * raw);
      if (dbias) atomicAdd(dbias + (W == 1 ? h : h * W + c), dx);
    }
  }
}

__global__ void zero_kernel(float* __restrict__ p, long n) {
  for (long i = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<long>(gridDim.x) * blockDim.x)
    p[i] = 0.f;
}

hipError_t zero(float* p, long n, hipStream_t s) {
  if (!p || n == 0) return hipSuccess;
  long blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  zero_kernel<<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s>>>(p, n);
  return hipGetLastError();
}

// the transforms' chain rule, if any transform is on
template <typename In>
hipError_t tf_bwd(const BwdArgs& a, const In* be, const In* de, long tokh, hipStream_t s) {
  if (!a.tf.A_log && !a.tf.beta_mode) return hipSuccess;
  const int W = a.decay_kind == DECAY_CHANNEL ? a.DK : 1;
  long blocks = (tokh * W + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  tf_bwd_kernel<In><<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s>>>(
      be, de, a.dbeta, a.tf.A_log ? a.ddecay : nullptr, a.dA_log, a.tf.dt_bias ? a.ddt_bias : nullptr,
      a.tf, a.H, W, tokh);
  return hipGetLastError();
}

template <typename In>
hipError_t dispatch_bwd(const BwdArgs& a, hipStream_t s) {
  const long qk = static_cast<long>(a.B) * a.T * a.Hk * a.DK;
  const long tokh = static_cast<long>(a.B) * a.T * a.H;
  // Every element of dv, dbeta and the decay's gradient is written; dq and
  // dk too unless value heads share q/k heads (then they are added up).
  hipError_t e = hipSuccess;
  if (a.H != a.Hk) {
    e = zero(a.dq, qk, s);
    if (e == hipSuccess) e = zero(a.dk, qk, s);
  }
  if (e == hipSuccess && a.tf.A_log) e = zero(a.dA_log, a.H, s);
  if (e == hipSuccess && a.tf.A_log && a.tf.dt_bias)
    e = zero(a.ddt_bias, a.decay_kind == DECAY_CHANNEL ? static_cast<long>(a.H) * a.DK : a.H, s);
  if (e != hipSuccess) return e;
  const In* q = static_cast<const In*>(a.q);
  const In* k = static_cast<const In*>(a.k);
  const In* be = static_cast<const In*>(a.beta);
  const In* de = static_cast<const In*>(a.decay);
  e = launch_bwd_chunked(a, s);
  if (e != hipSuccess) return e;
  // without grouped heads the chunked kernels have taken the norm's backward
  if (a.H == a.Hk) return tf_bwd(a, be, de, tokh, s);
  const long rows = static_cast<long>(a.B) * a.T * a.Hk;
  const dim3 g2(static_cast<unsigned>((2 * rows + 3) / 4)), b2(256);
  if (a.DK == 32) norm_bwd_kernel<32, In><<<g2, b2, 0, s>>>(q, k, a.dq, a.dk, rows, a.scale, a.l2norm);
  else if (a.DK == 64) norm_bwd_kernel<64, In><<<g2, b2, 0, s>>>(q, k, a.dq, a.dk, rows, a.scale, a.l2norm);
  else norm_bwd_kernel<128, In><<<g2, b2, 0, s>>>(q, k, a.dq, a.dk, rows, a.scale, a.l2norm);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return tf_bwd(a, be, de, tokh, s);
}

}  // namespace

size_t bwd_workspace_bytes(int B, int T, int H, int DK, int DV) {
  return bwd_chunked_workspace_bytes(B, T, H, DK, DV);
}

hipError_t launch_bwd(const BwdArgs& a, hipStream_t s) {
  return a.dtype == 0 ? dispatch_bwd<float>(a, s) : dispatch_bwd<bf16_t>(a, s);
}

}  // namespace kda
