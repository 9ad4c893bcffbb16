// Recurrent forward: the pure sequential scan of the gated delta rule
// (ejkernel kda, "Algorithm Modes", Recurrent), one workgroup per
// (batch, head) with the fp32 state resident in registers for the whole
// sequence.  Every token applies the one-step closed form
//   delta = beta (v - S^T k_hat),  o = S^T (exp(g) q_hat) + (q_hat . k_hat) delta,
//   S <- diag(exp(g)) S + k_hat delta^T.
// It is the GPU-side cross-check of the chunked path and a low-memory
// alternative to it, not a throughput path: its time grows with T dependent
// token steps.
#include "common.h"
#include "launch.h"

namespace kda {
namespace {

constexpr int kThreads = 256;
constexpr int kTB = 16;   // tokens staged in LDS at a time

template <int DK, int DV, typename In>
__global__ __launch_bounds__(kThreads) void recurrent_kernel(
    const In* __restrict__ q, const In* __restrict__ k, const In* __restrict__ v,
    const In* __restrict__ beta, const In* __restrict__ decay, int decay_kind,
    const float* __restrict__ init, float* __restrict__ o, float* __restrict__ state_out,
    int T, int H, float scale, int l2norm, Transforms tf, int Hk, int vfirst) {
  constexpr int CPW = DV / 4;           // value columns per wave
  constexpr int NCG = CPW / 4;          // float4 column groups per wave
  constexpr int NRG = 64 / NCG;         // row groups per wave
  constexpr int RPL = DK / NRG;         // state rows per lane
  static_assert(RPL >= 1 && DK % NRG == 0 && RPL % 1 == 0, "shape");
  constexpr int V = act<In>::kVec;
  constexpr int LPR = DK / V;           // lanes per token row in the staging loads

  __shared__ __align__(16) float s_q[kTB][DK];
  __shared__ __align__(16) float s_k[kTB][DK];
  __shared__ __align__(16) float s_g[kTB][DK];
  __shared__ __align__(16) float s_v[kTB][DV];
  __shared__ float s_b[kTB], s_qk[kTB], s_gh[kTB];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.x / H, h = blockIdx.x % H;
  const int cg = lane % NCG, rg = lane / NCG;
  const int col = wave * CPW + 4 * cg;          // first of this lane's 4 columns
  const int row0 = rg * RPL;                    // this lane's state rows row0 .. row0+RPL-1
  const long bh = static_cast<long>(b) * H + h;
  const int hk = h / (H / Hk);                  // q/k head of value head h
  // state element (key row c, value column n): key-major or value-major
  auto sidx = [&](int c, int n) {
    return bh * DK * DV + (vfirst ? static_cast<long>(n) * DK + c : static_cast<long>(c) * DV + n);
  };
  const float negA = tf.A_log ? -__expf(tf.A_log[h]) : 0.f;   // raw gate: -exp(A_log)

  f32x4 S[RPL];
#pragma unroll
  for (int i = 0; i < RPL; ++i) {
    if (init && !vfirst) S[i] = *reinterpret_cast<const f32x4*>(init + sidx(row0 + i, col));
    else if (init) S[i] = f32x4{init[sidx(row0 + i, col)], init[sidx(row0 + i, col + 1)],
                                init[sidx(row0 + i, col + 2)], init[sidx(row0 + i, col + 3)]};
    else S[i] = f32x4{0, 0, 0, 0};
  }

  for (int t0 = 0; t0 < T; t0 += kTB) {
    const int nt = min(kTB, T - t0);
    // Stage kTB tokens: normalised q, k, per-channel gate factors, v, beta.
    for (int idx = tid; idx < kTB * LPR; idx += kThreads) {
      const int tt = idx / LPR, seg = idx % LPR;
      float qv[V], kv[V];
      float sq = 0.f, sk = 0.f, sqk = 0.f;
      const bool live = tt < nt;
      const long base = ((static_cast<long>(b) * T + t0 + tt) * H + h) * DK + seg * V;
      const long kbase = ((static_cast<long>(b) * T + t0 + tt) * Hk + hk) * DK + seg * V;
      if (live) {
        act<In>::load_vec(q + kbase, qv);
        act<In>::load_vec(k + kbase, kv);
      } else {
#pragma unroll
        for (int e = 0; e < V; ++e) { qv[e] = 0.f; kv[e] = 0.f; }
      }
#pragma unroll
      for (int e = 0; e < V; ++e) { sq += qv[e] * qv[e]; sk += kv[e] * kv[e]; sqk += qv[e] * kv[e]; }
      // LPR consecutive lanes hold one token row (LPR divides 64 and idx ranges align).
      sq = group_sum<LPR>(sq); sk = group_sum<LPR>(sk); sqk = group_sum<LPR>(sqk);
      const float iq = (l2norm ? inv_norm(sq) : 1.f) * scale;
      const float ik = l2norm ? inv_norm(sk) : 1.f;
#pragma unroll
      for (int e = 0; e < V; ++e) {
        s_q[tt][seg * V + e] = qv[e] * iq;
        s_k[tt][seg * V + e] = kv[e] * ik;
      }
      if (decay_kind == DECAY_CHANNEL) {
        float gv[V];
        if (live) {
          act<In>::load_vec(decay + base, gv);
          if (tf.A_log) {
#pragma unroll
            for (int e = 0; e < V; ++e)
              gv[e] = gate_decay(gv[e], negA, tf.dt_bias ? tf.dt_bias[h * DK + seg * V + e] : 0.f,
                                 tf.lower);
          }
        } else {
#pragma unroll
          for (int e = 0; e < V; ++e) gv[e] = 0.f;
        }
#pragma unroll
        for (int e = 0; e < V; ++e) s_g[tt][seg * V + e] = __expf(gv[e]);
      }
      if (seg == 0) s_qk[tt] = sqk * iq * ik;
    }
    for (int idx = tid; idx < kTB * DV; idx += kThreads) {
      const int tt = idx / DV, n = idx % DV;
      s_v[tt][n] = tt < nt ? act<In>::load1(v + ((static_cast<long>(b) * T + t0 + tt) * H + h) * DV + n) : 0.f;
    }
    if (tid < kTB) {
      const bool live = tid < nt;
      const long tok = (static_cast<long>(b) * T + t0 + tid) * H + h;
      s_b[tid] = live ? beta_transform(act<In>::load1(beta + tok), tf.beta_mode) : 0.f;
      float gh = 0.f;
      if (decay_kind == DECAY_HEAD && live) {
        gh = act<In>::load1(decay + tok);
        if (tf.A_log) gh = gate_decay(gh, negA, tf.dt_bias ? tf.dt_bias[h] : 0.f, tf.lower);
      }
      s_gh[tid] = __expf(gh);
    }
    __syncthreads();

    for (int tt = 0; tt < nt; ++tt) {
      const float gh = s_gh[tt];
      f32x4 r = {0, 0, 0, 0}, y = {0, 0, 0, 0};
      float kc[RPL], gc[RPL];
#pragma unroll
      for (int i = 0; i < RPL; ++i) {
        kc[i] = s_k[tt][row0 + i];
        gc[i] = (decay_kind == DECAY_CHANNEL ? s_g[tt][row0 + i] : 1.f) * gh;
        const float qc = s_q[tt][row0 + i] * gc[i];
        r += S[i] * kc[i];
        y += S[i] * qc;
      }
#pragma unroll
      for (int off = NCG; off < 64; off <<= 1) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          r[e] += __shfl_xor(r[e], off, 64);
          y[e] += __shfl_xor(y[e], off, 64);
        }
      }
      const float bt = s_b[tt];
      f32x4 delta;
#pragma unroll
      for (int e = 0; e < 4; ++e) delta[e] = bt * (s_v[tt][col + e] - r[e]);
      if (rg == 0) {
        const f32x4 out = y + s_qk[tt] * delta;
        *reinterpret_cast<f32x4*>(o + ((static_cast<long>(b) * T + t0 + tt) * H + h) * DV + col) = out;
      }
#pragma unroll
      for (int i = 0; i < RPL; ++i) S[i] = S[i] * gc[i] + kc[i] * delta;
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < RPL; ++i) {
    if (!vfirst) {
      *reinterpret_cast<f32x4*>(state_out + sidx(row0 + i, col)) = S[i];
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) state_out[sidx(row0 + i, col + e)] = S[i][e];
    }
  }
}

template <typename In>
hipError_t dispatch(const FwdArgs& a, hipStream_t s) {
  const dim3 grid(a.B * a.H), block(kThreads);
  const In* q = static_cast<const In*>(a.q);
  const In* k = static_cast<const In*>(a.k);
  const In* v = static_cast<const In*>(a.v);
  const In* be = static_cast<const In*>(a.beta);
  const In* de = static_cast<const In*>(a.decay);
#define KDA_REC_CASE(dk, dv)                                                              \
  if (a.DK == dk && a.DV == dv) {                                                         \
    recurrent_kernel<dk, dv, In><<<grid, block, 0, s>>>(q, k, v, be, de, a.decay_kind,    \
                                                        a.init, a.o, a.state, a.T, a.H,   \
                                                        a.scale, a.l2norm, a.tf, a.Hk,    \
                                                        a.vfirst);                        \
    return hipGetLastError();                                                             \
  }
  KDA_REC_CASE(32, 32) KDA_REC_CASE(32, 64) KDA_REC_CASE(32, 128)
  KDA_REC_CASE(64, 32) KDA_REC_CASE(64, 64) KDA_REC_CASE(64, 128)
  KDA_REC_CASE(128, 32) KDA_REC_CASE(128, 64) KDA_REC_CASE(128, 128)
#undef KDA_REC_CASE
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_recurrent(const FwdArgs& a, hipStream_t s) {
  return a.dtype == 0 ? dispatch<float>(a, s) : dispatch<bf16_t>(a, s);
}

}  // namespace kda
