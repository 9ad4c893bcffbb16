// Backward of the gated delta rule: the gradients of (o, final state) with
// respect to q, k, v, beta, the decay and the initial state, given do and the
// final-state gradient (TileOPs "Linear Attention Operators",
// DeltaNetChunkBwdOp and GLAChunkBwdOp; kda-neuron-kernels README,
// kda_chunk_step_exact_bwd: dq, dk, dv, dg, dbeta, dstate_in).
//
// Reverse-mode differentiation of the recurrence, token by token (the
// forward: r = S^T k, delta = beta (v - r), S' = diag(a) S + k delta^T,
// o = S'^T q, a = exp(g), with q and k normalised and q scaled):
//
//   dS' += q do^T;  dq = S' do;  ddelta = dS'^T k;  dk = dS' delta - beta S ddelta
//   da = rowsum(dS' * S);  dbeta = ddelta . (v - r);  dv = beta ddelta
//   dS = diag(a) dS' - beta k ddelta^T
//
// Every value column of the state evolves on its own given q, k, beta and the
// decay, so a wave takes two (or, at DK = 32, four) columns, lanes over key
// channels, and interleaves their independent chains: the state columns and
// gradient columns sit in registers.  The reverse pass needs the
// state before every token: a first pass stores each column every 16 tokens
// in the workspace; the reverse pass recomputes the 16 states of a block into
// registers from there and steps back through them.  dv and the column's
// initial-state gradient belong to the wave alone; dq, dk, dbeta and the
// decay gradient are sums over columns.  Each wave stores its column's terms
// of dq, dk (and the per-channel decay gradient) in an LDS slice of its own;
// every 8 tokens the workgroup sums its four waves' slices and adds them to
// the outputs with one atomic add per element and workgroup (the order of
// those additions varies from run to run, within fp32 rounding).  LDS
// atomics, four waves adding to one address, cost about two thirds of the
// time when the sums were formed that way.  A last kernel carries dq and dk
// through the L2 norm and the scale.  All arithmetic is fp32.
//
// This is the plain form of the backward: time grows with T dependent
// token steps per column, and the work is not shaped for MFMA.
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace kda {
namespace {

constexpr int kBwdThreads = 256;   // four waves: four value columns of one (batch, head)
constexpr int kTB = 16;            // tokens per block (the checkpoint interval)
constexpr int kTH = kTB / 2;       // tokens per flush of the column sums
// value columns per wave: as many as fit two waves per SIMD without
// spilling much (256 registers; four columns spill 52 bytes a lane at
// DK = 64 and 648 at DK = 128, and run slower)
template <int DK> constexpr int ncw() { return DK >= 64 ? 2 : 4; }

template <int DK, int NCW, typename In>
struct BwdStage {
  float q[kTB][DK], k[kTB][DK], a[kTB][DK];   // normalised q (scaled), k; exp(decay) per channel
  float b[kTB], ah[kTB];                      // beta; exp(decay) per head
  float v[kTB][4 * NCW], dout[kTB][4 * NCW];  // v and do at the workgroup's columns
  // each wave's own column terms of dq, dk and the per-channel decay
  // gradient for half a block (plain stores), summed over the waves at each
  // half's end; per token the column sums of dbeta and the per-head decay
  // gradient
  float pq[4][kTH][DK], pk[4][kTH][DK], pg[4][kTH][DK];
  float db[kTB], dgh[kTB];
};

// NCW value columns per wave: their chains are independent, so a wave
// interleaves them; their terms of the column sums add up in registers.
template <int DK, int DV, int NCW, typename In>
__global__ __launch_bounds__(kBwdThreads, 2) void bwd_kernel(
    const In* __restrict__ q, const In* __restrict__ k, const In* __restrict__ v,
    const In* __restrict__ beta, const In* __restrict__ decay, int decay_kind,
    const float* __restrict__ init, const float* __restrict__ dout, const float* __restrict__ dfinal,
    float* __restrict__ dq, float* __restrict__ dk, float* __restrict__ dv, float* __restrict__ dbeta,
    float* __restrict__ ddecay, float* __restrict__ dinit, float* __restrict__ ckpt,
    int T, int H, int Hk, float scale, int l2norm, int vfirst, Transforms tf) {
  constexpr int CPL = (DK + 63) / 64;   // key channels per lane: c = lane + 64 e
  constexpr int V = act<In>::kVec;
  constexpr int LPR = DK / V;           // lanes per token row in the staging loads
  constexpr int NCG = 4 * NCW;          // columns per workgroup
  static_assert(DV % NCG == 0, "whole workgroups of columns");
  __shared__ BwdStage<DK, NCW, In> st;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ncg = DV / NCG;                                // workgroups per (b, h)
  const int bh = blockIdx.x / ncg;
  const int b = bh / H, h = bh % H;
  const int jg = (blockIdx.x % ncg) * NCG;                 // the workgroup's first column
  const int j0 = jg + wave * NCW;                          // this wave's first column
  const int hk = h / (H / Hk);
  const int nsub = (T + kTB - 1) / kTB;
  const bool chan = decay_kind == DECAY_CHANNEL, headd = decay_kind == DECAY_HEAD;
  bool live[CPL];
  int ch[CPL];
#pragma unroll
  for (int e = 0; e < CPL; ++e) {
    ch[e] = lane + 64 * e;
    live[e] = ch[e] < DK;
  }
  auto tok = [&](int t) { return static_cast<long>(b) * T + t; };
  // element (key row c, column jj) of an initial / final state
  auto sidx = [&](int c, int jj) {
    return vfirst ? (static_cast<long>(bh) * DV + jj) * DK + c : (static_cast<long>(bh) * DK + c) * DV + jj;
  };
  const float negA = tf.A_log ? -__expf(tf.A_log[h]) : 0.f;   // raw gate: -exp(A_log)
  // checkpoint of block n, column jj: [bh][n][column][DK]
  auto ck = [&](int n, int jj) { return ckpt + ((static_cast<long>(bh) * nsub + n) * DV + jj) * DK; };

  // Stage the tokens of block n: normalised q (scaled) and k, decay factors,
  // beta, and v (and with_do, do) at the workgroup's columns.
  auto stage = [&](int n, bool with_do) {
    const int t0 = n * kTB, nt = min(kTB, T - t0);
    for (int idx = tid; idx < kTB * LPR; idx += kBwdThreads) {
      const int tt = idx / LPR, seg = idx % LPR;
      float qv[V], kv[V];
      const bool in = tt < nt;
      const long kb = (tok(t0 + tt) * Hk + hk) * DK + seg * V;
      if (in) {
        act<In>::load_vec(q + kb, qv);
        act<In>::load_vec(k + kb, kv);
      } else {
#pragma unroll
        for (int e = 0; e < V; ++e) qv[e] = kv[e] = 0.f;
      }
      float sq = 0.f, sk = 0.f;
#pragma unroll
      for (int e = 0; e < V; ++e) { sq += qv[e] * qv[e]; sk += kv[e] * kv[e]; }
      sq = group_sum<LPR>(sq);
      sk = group_sum<LPR>(sk);
      const float iq = (l2norm ? inv_norm(sq) : 1.f) * scale;
      const float ik = l2norm ? inv_norm(sk) : 1.f;
      float gv[V];
      if (chan && in) {
        act<In>::load_vec(decay + (tok(t0 + tt) * H + h) * DK + seg * V, gv);
        if (tf.A_log) {
#pragma unroll
          for (int e = 0; e < V; ++e)
            gv[e] = gate_decay(gv[e], negA, tf.dt_bias ? tf.dt_bias[h * DK + seg * V + e] : 0.f, tf.lower);
        }
      } else {
#pragma unroll
        for (int e = 0; e < V; ++e) gv[e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < V; ++e) {
        st.q[tt][seg * V + e] = qv[e] * iq;
        st.k[tt][seg * V + e] = kv[e] * ik;
        st.a[tt][seg * V + e] = __expf(gv[e]);
      }
    }
    for (int idx = tid; idx < kTB * NCG; idx += kBwdThreads) {
      const int tt = idx / NCG, cw = idx % NCG;
      const bool in = tt < nt;
      const long vo = (tok(t0 + tt) * H + h) * DV + jg + cw;
      st.v[tt][cw] = in ? act<In>::load1(v + vo) : 0.f;
      st.dout[tt][cw] = (in && with_do) ? dout[vo] : 0.f;
    }
    if (tid < kTB) {
      const bool in = tid < nt;
      const long tk = tok(t0 + tid) * H + h;
      st.b[tid] = in ? beta_transform(act<In>::load1(beta + tk), tf.beta_mode) : 0.f;
      float gh = 0.f;
      if (headd && in) {
        gh = act<In>::load1(decay + tk);
        if (tf.A_log) gh = gate_decay(gh, negA, tf.dt_bias ? tf.dt_bias[h] : 0.f, tf.lower);
      }
      st.ah[tid] = __expf(gh);
    }
  };

  // ---- pass 1: the state columns at the start of every block ----
  float s[NCW][CPL];
#pragma unroll
  for (int w = 0; w < NCW; ++w) {
#pragma unroll
    for (int e = 0; e < CPL; ++e) s[w][e] = (init && live[e]) ? init[sidx(ch[e], j0 + w)] : 0.f;
  }
  for (int n = 0; n < nsub; ++n) {
    stage(n, false);
    __syncthreads();
#pragma unroll
    for (int w = 0; w < NCW; ++w) {
      float* c = ck(n, j0 + w);
#pragma unroll
      for (int e = 0; e < CPL; ++e)
        if (live[e]) c[ch[e]] = s[w][e];
    }
    const int t0 = n * kTB, nt = min(kTB, T - t0);
    for (int i = 0; i < nt; ++i) {
      float r[NCW];
#pragma unroll
      for (int w = 0; w < NCW; ++w) {
        r[w] = 0.f;
#pragma unroll
        for (int e = 0; e < CPL; ++e) r[w] += live[e] ? s[w][e] * st.k[i][ch[e]] : 0.f;
      }
#pragma unroll
      for (int w = 0; w < NCW; ++w) r[w] = dpp_group_sum<64>(r[w]);
#pragma unroll
      for (int w = 0; w < NCW; ++w) {
        const float delta = st.b[i] * (st.v[i][wave * NCW + w] - r[w]);
#pragma unroll
        for (int e = 0; e < CPL; ++e)
          if (live[e]) s[w][e] = (chan ? st.a[i][ch[e]] : st.ah[i]) * s[w][e] + st.k[i][ch[e]] * delta;
      }
    }
    __syncthreads();
  }

  // ---- pass 2: blocks in reverse ----
  float ds[NCW][CPL];
#pragma unroll
  for (int w = 0; w < NCW; ++w) {
#pragma unroll
    for (int e = 0; e < CPL; ++e) ds[w][e] = (dfinal && live[e]) ? dfinal[sidx(ch[e], j0 + w)] : 0.f;
  }
  for (int n = nsub - 1; n >= 0; --n) {
    stage(n, true);
    if (tid < kTB) st.db[tid] = st.dgh[tid] = 0.f;
    __syncthreads();
    const int t0 = n * kTB, nt = min(kTB, T - t0);
    // recompute the block's states: sp[i] enters token t0 + i
    float sp[kTB][NCW][CPL], rr[kTB][NCW];
#pragma unroll
    for (int w = 0; w < NCW; ++w) {
      const float* c = ck(n, j0 + w);
#pragma unroll
      for (int e = 0; e < CPL; ++e) s[w][e] = live[e] ? c[ch[e]] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < kTB; ++i) {
      if (i < nt) {
        float r[NCW];
#pragma unroll
        for (int w = 0; w < NCW; ++w) {
          r[w] = 0.f;
#pragma unroll
          for (int e = 0; e < CPL; ++e) {
            sp[i][w][e] = s[w][e];
            r[w] += live[e] ? s[w][e] * st.k[i][ch[e]] : 0.f;
          }
        }
#pragma unroll
        for (int w = 0; w < NCW; ++w) {
          rr[i][w] = dpp_group_sum<64>(r[w]);
          const float delta = st.b[i] * (st.v[i][wave * NCW + w] - rr[i][w]);
#pragma unroll
          for (int e = 0; e < CPL; ++e)
            if (live[e]) s[w][e] = (chan ? st.a[i][ch[e]] : st.ah[i]) * s[w][e] + st.k[i][ch[e]] * delta;
        }
      }
    }
    // The half block's column sums of dq, dk (and the per-channel decay
    // gradient), tokens t0 + hb .. t0 + hb + kTH - 1, into the outputs.
    auto flush = [&](int hb) {
      __syncthreads();
      for (int idx = tid; idx < kTH * DK; idx += kBwdThreads) {
        const int tt = idx / DK, cc = idx % DK;
        if (hb + tt < nt) {
          const long qo = (tok(t0 + hb + tt) * Hk + hk) * DK + cc;
          atomicAdd(dq + qo, (st.pq[0][tt][cc] + st.pq[1][tt][cc]) + (st.pq[2][tt][cc] + st.pq[3][tt][cc]));
          atomicAdd(dk + qo, (st.pk[0][tt][cc] + st.pk[1][tt][cc]) + (st.pk[2][tt][cc] + st.pk[3][tt][cc]));
          if (chan)
            atomicAdd(ddecay + (tok(t0 + hb + tt) * H + h) * DK + cc,
                      (st.pg[0][tt][cc] + st.pg[1][tt][cc]) + (st.pg[2][tt][cc] + st.pg[3][tt][cc]));
        }
      }
      __syncthreads();
    };
    // s now holds the states after the block
#pragma unroll
    for (int i = kTB - 1; i >= 0; --i) {
      if (i == kTH - 1) flush(kTH);
      if (i < nt) {
        const float bt = st.b[i];
        const float a0 = st.ah[i];
        float ddl[NCW], delta[NCW], dov[NCW];
        float dqv[CPL], dkv[CPL], dga[CPL];
#pragma unroll
        for (int e = 0; e < CPL; ++e) dqv[e] = dkv[e] = dga[e] = 0.f;
#pragma unroll
        for (int w = 0; w < NCW; ++w) {
          delta[w] = bt * (st.v[i][wave * NCW + w] - rr[i][w]);
          dov[w] = st.dout[i][wave * NCW + w];
          ddl[w] = 0.f;
#pragma unroll
          for (int e = 0; e < CPL; ++e) {
            const float snew = i + 1 < nt ? sp[i + 1 < kTB ? i + 1 : i][w][e] : s[w][e];
            if (live[e]) {
              ds[w][e] += st.q[i][ch[e]] * dov[w];
              dqv[e] += snew * dov[w];
              ddl[w] += ds[w][e] * st.k[i][ch[e]];
            }
          }
        }
#pragma unroll
        for (int w = 0; w < NCW; ++w) ddl[w] = dpp_group_sum<64>(ddl[w]);
        float dgs = 0.f, dbs = 0.f;
#pragma unroll
        for (int w = 0; w < NCW; ++w) {
#pragma unroll
          for (int e = 0; e < CPL; ++e) {
            if (live[e]) {
              const float a = chan ? st.a[i][ch[e]] : a0;
              dkv[e] += ds[w][e] * delta[w] - bt * ddl[w] * sp[i][w][e];
              const float g1 = ds[w][e] * sp[i][w][e] * a;   // d(decay) = a * da
              dga[e] += g1;
              dgs += g1;
              ds[w][e] = a * ds[w][e] - bt * ddl[w] * st.k[i][ch[e]];
            }
          }
          dbs += ddl[w] * (st.v[i][wave * NCW + w] - rr[i][w]);
        }
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
          if (live[e]) {
            st.pq[wave][i % kTH][ch[e]] = dqv[e];
            st.pk[wave][i % kTH][ch[e]] = dkv[e];
            if (chan) st.pg[wave][i % kTH][ch[e]] = dga[e];
          }
        }
        if (headd) dgs = dpp_group_sum<64>(dgs);
        if (lane == 0) {
          atomicAdd(&st.db[i], dbs);
          if (headd) atomicAdd(&st.dgh[i], dgs);
        }
        if (lane < NCW) {
          // lane w stores column j0 + w's dv
          float dvw = 0.f;
#pragma unroll
          for (int w = 0; w < NCW; ++w) dvw = lane == w ? bt * ddl[w] : dvw;
          dv[(tok(t0 + i) * H + h) * DV + j0 + lane] = dvw;
        }
      }
    }
    flush(0);
    if (tid < nt) {
      atomicAdd(dbeta + tok(t0 + tid) * H + h, st.db[tid]);
      if (headd) atomicAdd(ddecay + tok(t0 + tid) * H + h, st.dgh[tid]);
    }
    __syncthreads();
  }
  if (dinit) {
#pragma unroll
    for (int w = 0; w < NCW; ++w) {
#pragma unroll
      for (int e = 0; e < CPL; ++e)
        if (live[e]) dinit[sidx(ch[e], j0 + w)] = ds[w][e];
    }
  }
}

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

template <typename In>
hipError_t dispatch_bwd(const BwdArgs& a, hipStream_t s) {
  const long qk = static_cast<long>(a.B) * a.T * a.Hk * a.DK;
  const long tokh = static_cast<long>(a.B) * a.T * a.H;
  // The chunked form writes every element of dbeta and of a per-head
  // ddecay, and of dq and dk unless value heads share q/k heads (then it
  // adds); the token-by-token form adds into all of them.
  const bool chunked = a.decay_kind != DECAY_CHANNEL;
  hipError_t e = hipSuccess;
  if (!chunked || a.H != a.Hk) {
    e = zero(a.dq, qk, s);
    if (e == hipSuccess) e = zero(a.dk, qk, s);
  }
  if (e == hipSuccess && !chunked) e = zero(a.dbeta, tokh, s);
  if (e == hipSuccess && a.decay_kind == DECAY_CHANNEL) e = zero(a.ddecay, tokh * a.DK, s);
  if (e == hipSuccess && a.tf.A_log) e = zero(a.dA_log, a.H, s);
  if (e == hipSuccess && a.tf.A_log && a.tf.dt_bias)
    e = zero(a.ddt_bias, a.decay_kind == DECAY_CHANNEL ? static_cast<long>(a.H) * a.DK : a.H, s);
  if (e != hipSuccess) return e;
  const In* q = static_cast<const In*>(a.q);
  const In* k = static_cast<const In*>(a.k);
  const In* v = static_cast<const In*>(a.v);
  const In* be = static_cast<const In*>(a.beta);
  const In* de = static_cast<const In*>(a.decay);
  const dim3 block(kBwdThreads);
  bool launched = false;
  if (chunked) {
    e = launch_bwd_chunked(a, s);
    if (e != hipSuccess) return e;
    launched = true;
  }
#define KDA_BWD_CASE(dk_, dv_)                                                                   \
  if (!launched && a.DK == dk_ && a.DV == dv_) {                                                 \
    bwd_kernel<dk_, dv_, ncw<dk_>(), In><<<dim3(a.B * a.H * (dv_ / (4 * ncw<dk_>()))), block, 0, s>>>(q, k, v, be, de, a.decay_kind, a.init, a.dout, \
                                                    a.dfinal, a.dq, a.dk, a.dv, a.dbeta,         \
                                                    a.ddecay, a.dinit, a.ckpt, a.T, a.H, a.Hk,   \
                                                    a.scale, a.l2norm, a.vfirst, a.tf);          \
    launched = true;                                                                             \
  }
  KDA_BWD_CASE(32, 32) KDA_BWD_CASE(32, 64) KDA_BWD_CASE(32, 128)
  KDA_BWD_CASE(64, 32) KDA_BWD_CASE(64, 64) KDA_BWD_CASE(64, 128)
  KDA_BWD_CASE(128, 32) KDA_BWD_CASE(128, 64) KDA_BWD_CASE(128, 128)
#undef KDA_BWD_CASE
  if (!launched) return hipErrorInvalidValue;
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long rows = static_cast<long>(a.B) * a.T * a.Hk;
  const dim3 g2(static_cast<unsigned>((2 * rows + 3) / 4)), b2(256);
  if (a.DK == 32) norm_bwd_kernel<32, In><<<g2, b2, 0, s>>>(q, k, a.dq, a.dk, rows, a.scale, a.l2norm);
  else if (a.DK == 64) norm_bwd_kernel<64, In><<<g2, b2, 0, s>>>(q, k, a.dq, a.dk, rows, a.scale, a.l2norm);
  else norm_bwd_kernel<128, In><<<g2, b2, 0, s>>>(q, k, a.dq, a.dk, rows, a.scale, a.l2norm);
  e = hipGetLastError();
  if (e != hipSuccess || (!a.tf.A_log && !a.tf.beta_mode)) return e;
  const int W = a.decay_kind == DECAY_CHANNEL ? a.DK : 1;
  long blocks = (tokh * W + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  tf_bwd_kernel<In><<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s>>>(
      be, de, a.dbeta, a.tf.A_log ? a.ddecay : nullptr, a.dA_log, a.tf.dt_bias ? a.ddt_bias : nullptr,
      a.tf, a.H, W, tokh);
  return hipGetLastError();
}

}  // namespace

size_t bwd_workspace_bytes(int B, int T, int H, int DK, int DV) {
  const long nsub = (static_cast<long>(T) + kTB - 1) / kTB;
  const size_t plain = static_cast<size_t>(B) * H * nsub * DV * DK * sizeof(float);
  return std::max(plain, bwd_chunked_workspace_bytes(B, T, H, DK, DV));
}

hipError_t launch_bwd(const BwdArgs& a, hipStream_t s) {
  return a.dtype == 0 ? dispatch_bwd<float>(a, s) : dispatch_bwd<bf16_t>(a, s);
}

}  // namespace kda
