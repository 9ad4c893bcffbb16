// Single-token decode: one step of the gated delta rule for every (batch, head),
// the fp32 state streamed from HBM and written back in place.
//
// Closed form of one step (TileOPs "Linear Attention Operators",
// DeltaNetRecurrentFwdOp, with the ejkernel recurrence's gate on the state):
//   r     = S^T k_hat                  (read of the undecayed state)
//   delta = beta (v - r)
//   o     = S^T (exp(g) * q_hat) + (q_hat . k_hat) delta
//   S'    = diag(exp(g)) S + k_hat delta^T
// so the whole step needs one read and one write of S.  The kernel is bound
// by HBM bandwidth: 2 * DK * DV * 4 bytes of state traffic per (batch, head)
// against about 6 * DK * DV flops.  Every value column is independent given
// the token vectors; the reductions run over key rows.  A workgroup holds one
// (batch, head)'s state in registers (64 KB at DK = DV = 128), read and
// written in contiguous whole rows (key-major) or whole columns (value-major).
#include "common.h"
#include "launch.h"

namespace kda {
namespace {

constexpr int kThreads = 256;

// Columns per workgroup of the value-major kernel: at least one pass of
// DK / 4-lane columns, at most 32.
template <int DK, int DV> constexpr int decode_vm_cols() {
  return DV < 32 ? DV : (32 > 1024 / DK ? 32 : 1024 / DK);
}

// Key-major state [.., DK, DV]: a workgroup of NW waves takes one (batch,
// head), wave w the key rows w DK/NW .. (w + 1) DK/NW - 1 with all DV columns.
// A lane holds a float4 of columns in rows rg + NRG i of the wave's block, so
// one wave instruction reads NRG whole rows, contiguous in memory.  The two
// reductions over rows run inside the wave (lane-swap and DPP moves), then
// over the waves through LDS behind the workgroup's one barrier.  Every
// wave forms the token vectors' norms itself from all DK entries.
// Waves per workgroup of the key-major kernel: eight where the rows allow
// (at DK = DV = 128: 16 rows, 8 float4 registers of state per lane; four
// waves with 32 rows each measured 0.709 of HBM against 0.712-0.720, sixteen
// waves 0.63)
template <int DK, int DV> constexpr int decode_waves() {
  return DK / (256 / DV) >= 8 ? 8 : DK / (256 / DV);
}
template <int DK, int DV, typename In>
__global__ __launch_bounds__(512) void decode_kernel(
    const In* __restrict__ q, const In* __restrict__ k, const In* __restrict__ v,
    const In* __restrict__ beta, const In* __restrict__ decay, int decay_kind,
    float* __restrict__ state, float* __restrict__ o, float scale, int l2norm, int H,
    Transforms tf, int Hk) {
  constexpr int NW = decode_waves<DK, DV>();
  constexpr int RW = DK / NW;             // key rows per wave
  constexpr int NC4 = DV / 4;             // float4 column groups: lanes per row
  constexpr int NRG = 64 / NC4;           // rows per wave instruction
  constexpr int RPT = RW / NRG;           // rows per lane
  static_assert(RPT >= 1 && RW % NRG == 0 && (NC4 == 8 || NC4 == 16 || NC4 == 32), "shape");

  __shared__ float s_q[DK], s_k[DK], s_gate[DK];
  __shared__ f32x4 s_r[NW][NC4], s_y[NW][NC4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const long bh = blockIdx.x;
  const int cg = lane % NC4, rg = lane / NC4;
  const int r0 = wave * RW;
  float* S = state + bh * DK * DV;
  const int h = static_cast<int>(bh % H);
  const long bhk = (bh / H) * Hk + h / (H / Hk);
  const float negA = tf.A_log ? -__expf(tf.A_log[h]) : 0.f;

  f32x4 st[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i)
    st[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S + (r0 + rg + NRG * i) * DV) + cg);

  // the token vectors, whole, in every wave (the same values to the same LDS
  // words), and their norms
  float pq = 0.f, pk = 0.f, pqk = 0.f;
#pragma unroll
  for (int c = lane; c < DK; c += 64) {
    const float qc = act<In>::load1(q + bhk * DK + c);
    const float kc = act<In>::load1(k + bhk * DK + c);
    s_q[c] = qc;
    s_k[c] = kc;
    float gc = 1.f;
    if (decay_kind == DECAY_CHANNEL) {
      float g = act<In>::load1(decay + bh * DK + c);
      if (tf.A_log) g = gate_decay(g, negA, tf.dt_bias ? tf.dt_bias[h * DK + c] : 0.f, tf.lower);
      gc = __expf(g);
    }
    s_gate[c] = gc;
    pq += qc * qc; pk += kc * kc; pqk += qc * kc;
  }
  pq = group_sum<64>(pq); pk = group_sum<64>(pk); pqk = group_sum<64>(pqk);
  const float iq = (l2norm ? inv_norm(pq) : 1.f) * scale;
  const float ik = l2norm ? inv_norm(pk) : 1.f;
  const float qk = pqk * iq * ik;
  const float b = beta_transform(act<In>::load1(beta + bh), tf.beta_mode);
  float ghead = 1.f;
  if (decay_kind == DECAY_HEAD) {
    float g = act<In>::load1(decay + bh);
    if (tf.A_log) g = gate_decay(g, negA, tf.dt_bias ? tf.dt_bias[h] : 0.f, tf.lower);
    ghead = __expf(g);
  }
  // the wave's own LDS writes land before its lanes read each other's
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_wave_barrier();

  f32x4 r = {0, 0, 0, 0}, y = {0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int c = r0 + rg + NRG * i;
    const float kc = s_k[c] * ik;
    const float qc = s_q[c] * iq * s_gate[c] * ghead;
    r += st[i] * kc;
    y += st[i] * qc;
  }
  // over the wave's row groups (lanes with equal lane % NC4: at NC4 = 32 the
  // two halves of the wave), then the waves
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if constexpr (NC4 == 32) {
      r[e] = xor32_sum(r[e]);
      y[e] = xor32_sum(y[e]);
    } else {
      r[e] = rowgroup_sum<NC4>(r[e]);
      y[e] = rowgroup_sum<NC4>(y[e]);
    }
  }
  if (rg == 0) {
    s_r[wave][cg] = r;
    s_y[wave][cg] = y;
  }
  __syncthreads();
  r = s_r[0][cg];
  y = s_y[0][cg];
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    r += s_r[w][cg];
    y += s_y[w][cg];
  }
  float vc[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) vc[e] = act<In>::load1(v + bh * DV + 4 * cg + e);
  f32x4 delta;
#pragma unroll
  for (int e = 0; e < 4; ++e) delta[e] = b * (vc[e] - r[e]);
  if (wave == 0 && rg == 0) *reinterpret_cast<f32x4*>(o + bh * DV + 4 * cg) = y + qk * delta;
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int c = r0 + rg + NRG * i;
    const float gc = s_gate[c] * ghead;
    const float kc = s_k[c] * ik;
    const f32x4 ns = st[i] * gc + kc * delta;
    __builtin_nontemporal_store(ns, reinterpret_cast<f32x4*>(S + c * DV) + cg);
  }
}

// Value-major state [.., DV, DK] (each value column's DK key rows
// contiguous): a workgroup takes CS value columns of one (batch, head); DK / 4
// consecutive lanes hold one column as float4s, so loads and stores stay
// contiguous, and the two column reductions run over those lanes with DPP.
template <int DK, int DV, typename In>
__global__ __launch_bounds__(kThreads) void decode_vm_kernel(
    const In* __restrict__ q, const In* __restrict__ k, const In* __restrict__ v,
    const In* __restrict__ beta, const In* __restrict__ decay, int decay_kind,
    float* __restrict__ state, float* __restrict__ o, float scale, int l2norm, int H,
    Transforms tf, int Hk) {
  constexpr int CS = decode_vm_cols<DK, DV>();
  constexpr int NSPLIT = DV / CS;
  constexpr int LPC = DK / 4;             // lanes per value column
  constexpr int CPP = kThreads / LPC;     // columns per pass
  constexpr int CPT = CS / CPP;           // columns per thread
  static_assert(CPT >= 1 && CS % CPP == 0 && 64 % LPC == 0, "shape");
  constexpr int NW = kThreads / 64;

  __shared__ float s_q[DK], s_k[DK], s_gate[DK], s_v[CS];
  __shared__ float s_red[3][NW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const long bh = blockIdx.x / NSPLIT;
  const int n0 = (blockIdx.x % NSPLIT) * CS;
  const int cq = tid % LPC, cr = tid / LPC;   // key rows 4 cq .. 4 cq + 3 of columns cr + CPP i
  float* S = state + bh * DK * DV + static_cast<long>(n0) * DK;
  const int h = static_cast<int>(bh % H);
  const long bhk = (bh / H) * Hk + h / (H / Hk);
  const float negA = tf.A_log ? -__expf(tf.A_log[h]) : 0.f;

  f32x4 st[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i)
    st[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S + (cr + CPP * i) * DK) + cq);

  float pq = 0.f, pk = 0.f, pqk = 0.f;
  for (int c = tid; c < DK; c += kThreads) {
    const float qc = act<In>::load1(q + bhk * DK + c);
    const float kc = act<In>::load1(k + bhk * DK + c);
    s_q[c] = qc;
    s_k[c] = kc;
    float gc = 1.f;
    if (decay_kind == DECAY_CHANNEL) {
      float g = act<In>::load1(decay + bh * DK + c);
      if (tf.A_log) g = gate_decay(g, negA, tf.dt_bias ? tf.dt_bias[h * DK + c] : 0.f, tf.lower);
      gc = __expf(g);
    }
    s_gate[c] = gc;
    pq += qc * qc; pk += kc * kc; pqk += qc * kc;
  }
  for (int n = tid; n < CS; n += kThreads) s_v[n] = act<In>::load1(v + bh * DV + n0 + n);
  pq = group_sum<64>(pq); pk = group_sum<64>(pk); pqk = group_sum<64>(pqk);
  if (lane == 0) { s_red[0][wave] = pq; s_red[1][wave] = pk; s_red[2][wave] = pqk; }
  __syncthreads();
  float sq = 0.f, sk = 0.f, sqk = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) { sq += s_red[0][w]; sk += s_red[1][w]; sqk += s_red[2][w]; }
  const float iq = (l2norm ? inv_norm(sq) : 1.f) * scale;
  const float ik = l2norm ? inv_norm(sk) : 1.f;
  const float qk = sqk * iq * ik;
  const float b = beta_transform(act<In>::load1(beta + bh), tf.beta_mode);
  float ghead = 1.f;
  if (decay_kind == DECAY_HEAD) {
    float g = act<In>::load1(decay + bh);
    if (tf.A_log) g = gate_decay(g, negA, tf.dt_bias ? tf.dt_bias[h] : 0.f, tf.lower);
    ghead = __expf(g);
  }

  // this thread's four key rows
  f32x4 kc, qg, gc;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int c = 4 * cq + e;
    kc[e] = s_k[c] * ik;
    gc[e] = s_gate[c] * ghead;
    qg[e] = s_q[c] * iq * gc[e];
  }
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int n = cr + CPP * i;
    float r = st[i][0] * kc[0] + st[i][1] * kc[1] + st[i][2] * kc[2] + st[i][3] * kc[3];
    float y = st[i][0] * qg[0] + st[i][1] * qg[1] + st[i][2] * qg[2] + st[i][3] * qg[3];
    r = dpp_group_sum<LPC>(r);
    y = dpp_group_sum<LPC>(y);
    const float delta = b * (s_v[n] - r);
    if (cq == 0) o[bh * DV + n0 + n] = y + qk * delta;
    const f32x4 ns = st[i] * gc + kc * delta;
    __builtin_nontemporal_store(ns, reinterpret_cast<f32x4*>(S + n * DK) + cq);
  }
}

template <typename In>
hipError_t dispatch(const FwdArgs& a, hipStream_t s) {
  const dim3 block(kThreads);
  const In* q = static_cast<const In*>(a.q);
  const In* k = static_cast<const In*>(a.k);
  const In* v = static_cast<const In*>(a.v);
  const In* be = static_cast<const In*>(a.beta);
  const In* de = static_cast<const In*>(a.decay);
#define KDA_DECODE_CASE(dk, dv)                                                              \
  if (a.DK == dk && a.DV == dv) {                                                            \
    const dim3 grid(a.B * a.H * (dv / decode_vm_cols<dk, dv>()));                            \
    if (a.vfirst)                                                                            \
      decode_vm_kernel<dk, dv, In><<<grid, block, 0, s>>>(q, k, v, be, de, a.decay_kind,     \
                                                          a.state, a.o, a.scale, a.l2norm,   \
                                                          a.H, a.tf, a.Hk);                  \
    else                                                                                     \
      decode_kernel<dk, dv, In><<<dim3(a.B * a.H), dim3(64 * decode_waves<dk, dv>()), 0, s>>>(\
          q, k, v, be, de, a.decay_kind, a.state, a.o, a.scale, a.l2norm, a.H, a.tf, a.Hk);  \
    return hipGetLastError();                                                                \
  }
  KDA_DECODE_CASE(32, 32) KDA_DECODE_CASE(32, 64) KDA_DECODE_CASE(32, 128)
  KDA_DECODE_CASE(64, 32) KDA_DECODE_CASE(64, 64) KDA_DECODE_CASE(64, 128)
  KDA_DECODE_CASE(128, 32) KDA_DECODE_CASE(128, 64) KDA_DECODE_CASE(128, 128)
#undef KDA_DECODE_CASE
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(const FwdArgs& a, hipStream_t s) {
  return a.dtype == 0 ? dispatch<float>(a, s) : dispatch<bf16_t>(a, s);
}

}  // namespace kda
