// Chunked backward of the gated delta rule for a per-head (scalar) decay or
// none: the gradients of (o, final state) with respect to q, k, v, beta, the
// decay and the initial state, the same quantities as the token-by-token
// backward (backward.hip), computed chunk by chunk in the WY form that the
// forward uses (TileOPs "Linear Attention Operators": the DeltaNet chunked
// pipeline and its DeltaNetChunkBwdOp, GLAChunkBwdOp for the decay).
//
// For a chunk of C tokens entering with state S0, with q, k the normalised
// (q scaled) rows, gam the inclusive and gx the exclusive in-chunk cumulative
// log decay, gC the chunk's total and F = exp(gC - gam):
//
//   A = diag(beta) (K K^T . W), W_rs = exp(gx_r - gam_s) on s < r;  T = (I + A)^-1
//   X = V - exp(gx) . K S0;  Y = diag(beta) X;  D = T Y
//   P = (Q K^T) . Vw, Vw_rs = exp(gam_r - gam_s) on s <= r
//   O = exp(gam) . Q S0 + P D;   S1 = exp(gC) S0 + K^T (F . D)
//
// Every exponent is <= 0.  Pulling back (dO, dS1), dS1 the gradient of the
// chunk's final state:
//
//   dD = P^T dO + F . K dS1;  dY = T^T dD;  dX = beta . dY (= dv)
//   dS0 = exp(gC) dS1 + Q^T (exp(gam) . dO) - K^T (exp(gx) . dX)
//   dT = dD Y^T;  dA = -(T^T dT T^T) on A's support;  dP = dO D^T on P's
//   dbeta_r = sum_n dY_rn X_rn + sum_s dA_rs (K K^T)_rs W_rs
//   dq = exp(gam) . dO S0^T + Z K,                       Z = dP . Vw
//   dk = -exp(gx) . dX S0^T + F . D dS1^T + (dG + dG^T) K + Z^T Q,  dG = diag(beta) dA . W
//   and the decay through gam, gx and gC (each exponential's own factor),
//   dg_t = sum_{r >= t} dgam_r + sum_{r > t} dgx_r + dgC.
//
// Four kernels: (0) per chunk, in parallel: the rows' norm factors, beta,
// the cumulative decays, T and P; (1) per (b, h, kNS value columns): the
// walk over the chunks storing each chunk's S0; (2) the same slices in
// reverse: the walk of the state gradient storing each chunk's dS1 and
// writing dv and the initial state's gradient; (3) per chunk, in parallel:
// everything else, over the value columns kNS at a time.  The q and k
// gradients are those of the normalised rows; the norm's backward runs after,
// as for the token-by-token form.  All arithmetic is fp32.
#include "common.h"
#include "launch.h"

namespace kda {
namespace {

constexpr int kC = 32;        // tokens per chunk
constexpr int kNS = 16;       // value columns per slice
constexpr int kThr = 256;     // prep and walk workgroups
constexpr int kThr3 = 512;    // local-gradient workgroups

// Workspace carve (floats): per token-head, per chunk-head matrix, per
// chunk-head state.
struct CWs {
  float *sq, *sk, *bt, *gm, *gx;   // [B*T*H]: norm factors of q and k, beta, gam, gx
  float *Tm, *Pm;                  // [B*H*N][C][C]
  float *S0, *dS1;                 // [B*H*N][DK][DV]
};

size_t align_f(size_t n) { return (n + 63) & ~static_cast<size_t>(63); }

size_t ws_floats(int B, int T, int H, int DK, int DV, CWs* w, float* base) {
  const size_t tok = align_f(static_cast<size_t>(B) * T * H);
  const size_t N = (static_cast<size_t>(T) + kC - 1) / kC;
  const size_t ch = static_cast<size_t>(B) * H * N;
  const size_t mats = align_f(ch * kC * kC), st = ch * DK * DV;
  if (w) {
    float* p = base;
    w->sq = p; p += tok;
    w->sk = p; p += tok;
    w->bt = p; p += tok;
    w->gm = p; p += tok;
    w->gx = p; p += tok;
    w->Tm = p; p += mats;
    w->Pm = p; p += mats;
    w->S0 = p; p += st;
    w->dS1 = p;
  }
  return 5 * tok + 2 * mats + 2 * st;
}

// (0) per (b, h, chunk): the norm factors of the rows, beta and the
// cumulative decays per token; T and P of the chunk.
template <int DK, typename In>
__global__ __launch_bounds__(kThr) void cbwd_prep(const In* __restrict__ q, const In* __restrict__ k,
                                                  const In* __restrict__ beta, const In* __restrict__ decay,
                                                  int headd, CWs w, int T, int H, int Hk, int N, float scale,
                                                  int l2norm, Transforms tf) {
  __shared__ float kh[kC][DK + 1], qh[kC][DK + 1];
  __shared__ float sA[kC][kC + 1];
  __shared__ float sbt[kC], sgm[kC], sgx[kC];
  const int tid = threadIdx.x;
  const int ci = blockIdx.x % N, bh = blockIdx.x / N, b = bh / H, h = bh % H, hk = h / (H / Hk);
  const int t0 = ci * kC, L = min(kC, T - t0);
  const long tok0 = static_cast<long>(b) * T + t0;
  {
    // eight lanes to a row
    constexpr int SEG = DK / 8;
    const int r = tid / 8, sg = tid % 8;
    const bool in = r < L;
    const long base = ((tok0 + r) * Hk + hk) * DK + sg * SEG;
    float qv[SEG], kv[SEG], sq = 0.f, sk = 0.f;
#pragma unroll
    for (int e = 0; e < SEG; ++e) {
      qv[e] = in ? act<In>::load1(q + base + e) : 0.f;
      kv[e] = in ? act<In>::load1(k + base + e) : 0.f;
      sq += qv[e] * qv[e];
      sk += kv[e] * kv[e];
    }
    sq = dpp_group_sum<8>(sq);
    sk = dpp_group_sum<8>(sk);
    const float fq = (l2norm ? inv_norm(sq) : 1.f) * scale, fk = l2norm ? inv_norm(sk) : 1.f;
#pragma unroll
    for (int e = 0; e < SEG; ++e) {
      qh[r][sg * SEG + e] = qv[e] * fq;
      kh[r][sg * SEG + e] = kv[e] * fk;
    }
    if (sg == 0 && in) {
      w.sq[(tok0 + r) * H + h] = fq;
      w.sk[(tok0 + r) * H + h] = fk;
    }
  }
  if (tid < kC) {
    // token r in lane r of wave 0: beta, the decay and its scan
    const int r = tid;
    const bool in = r < L;
    const long ti = (tok0 + r) * H + h;
    const float bt = in ? beta_transform(act<In>::load1(beta + ti), tf.beta_mode) : 0.f;
    float g = 0.f;
    if (headd && in) {
      g = act<In>::load1(decay + ti);
      if (tf.A_log) g = gate_decay(g, -__expf(tf.A_log[h]), tf.dt_bias ? tf.dt_bias[h] : 0.f, tf.lower);
    }
    float gam = g;
#pragma unroll
    for (int off = 1; off < kC; off <<= 1) {
      const float y = __shfl_up(gam, off, kC);
      if (r >= off) gam += y;
    }
    float gx = __shfl_up(gam, 1, kC);
    if (r == 0) gx = 0.f;
    sbt[r] = bt;
    sgm[r] = gam;
    sgx[r] = gx;
    if (in) {
      w.bt[ti] = bt;
      w.gm[ti] = gam;
      w.gx[ti] = gx;
    }
  }
  __syncthreads();
  const size_t cb = (static_cast<size_t>(bh) * N + ci) * kC * kC;
  for (int idx = tid; idx < kC * kC; idx += kThr) {
    const int r = idx / kC, s = idx % kC;
    float gkk = 0.f, gqk = 0.f;
#pragma unroll 8
    for (int c = 0; c < DK; ++c) {
      gkk += kh[r][c] * kh[s][c];
      gqk += qh[r][c] * kh[s][c];
    }
    sA[r][s] = s < r ? sbt[r] * gkk * __expf(sgx[r] - sgm[s]) : 0.f;
    w.Pm[cb + idx] = s <= r ? gqk * __expf(sgm[r] - sgm[s]) : 0.f;
  }
  __syncthreads();
  if (tid < kC) {
    // column j of T = (I + A)^-1 by forward substitution
    const int j = tid;
    float x[kC];
#pragma unroll
    for (int r = 0; r < kC; ++r) {
      float acc = r == j ? 1.f : 0.f;
#pragma unroll
      for (int s = 0; s < r; ++s) acc -= sA[r][s] * x[s];
      x[r] = acc;
    }
#pragma unroll
    for (int r = 0; r < kC; ++r) w.Tm[cb + r * kC + j] = x[r];
  }
}

// Per-chunk token factors: beta, exp(gx), exp(gam), F = exp(gC - gam), all
// zero past the sequence's end, and exp(gC).
struct TokVec {
  float bt[kC], egx[kC], egm[kC], F[kC];
  float egC;
};
__device__ __forceinline__ void load_tokvec(TokVec& tv, const CWs& w, long tok0, int H, int h, int L, int tid) {
  if (tid < kC) {
    const int r = tid;
    const bool in = r < L;
    const long t = (tok0 + r) * H + h;
    const float gC = w.gm[(tok0 + L - 1) * H + h];
    tv.bt[r] = in ? w.bt[t] : 0.f;
    tv.egx[r] = in ? __expf(w.gx[t]) : 0.f;
    tv.egm[r] = in ? __expf(w.gm[t]) : 0.f;
    tv.F[r] = in ? __expf(gC - w.gm[t]) : 0.f;
    if (r == 0) tv.egC = __expf(gC);
  }
}

// The normalised rows of a chunk (raw rows times their norm factor) into
// LDS rows of pitch KP; rows past the sequence's end are zero.
template <int DK, int KP, typename In>
__device__ __forceinline__ void stage_rows(float (*dst)[KP], const In* src, const float* fac, long tok0, int H,
                                           int h, int Hk, int hk, int L, int tid, int nthr) {
  constexpr int V = act<In>::kVec, LPR = DK / V;
  for (int idx = tid; idx < kC * LPR; idx += nthr) {
    const int r = idx / LPR, seg = idx % LPR;
    float x[V];
    if (r < L) {
      act<In>::load_vec(src + ((tok0 + r) * Hk + hk) * DK + seg * V, x);
      const float f = fac[(tok0 + r) * H + h];
#pragma unroll
      for (int e = 0; e < V; ++e) x[e] *= f;
    } else {
#pragma unroll
      for (int e = 0; e < V; ++e) x[e] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < V; ++e) dst[r][seg * V + e] = x[e];
  }
}

// T (and with Pd, P) of a chunk into LDS, one 16-byte load per thread and pass
__device__ __forceinline__ void stage_mats(float (*Td)[kC + 1], float (*Pd)[kC + 1], const CWs& w, size_t cb,
                                           int tid, int nthr) {
  for (int idx = tid; idx < kC * kC / 4; idx += nthr) {
    const int r = idx / (kC / 4), c4 = (idx % (kC / 4)) * 4;
    const f32x4 t = *reinterpret_cast<const f32x4*>(w.Tm + cb + r * kC + c4);
#pragma unroll
    for (int e = 0; e < 4; ++e) Td[r][c4 + e] = t[e];
    if (Pd) {
      const f32x4 p = *reinterpret_cast<const f32x4*>(w.Pm + cb + r * kC + c4);
#pragma unroll
      for (int e = 0; e < 4; ++e) Pd[r][c4 + e] = p[e];
    }
  }
}

// acc += A (16 x 4) B (4 x 16), fp32: lane l gives A[l % 16][l / 16] and
// B[l / 16][l % 16]; it holds rows 4 (l / 16) + j, j = 0..3, of column l % 16.
__device__ __forceinline__ f32x4 mma4(float a, float b, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
}

// (1) per (b, h, slice of kNS value columns): every chunk's S0 into the
// workspace, chunk after chunk.  The slice of the state (DK x 16) sits in
// MFMA accumulators, 16 key rows per tile, tile m in wave m % 4.  Per chunk:
// K S as partial products of each wave's own tiles (the tile is the B
// operand as it stands), summed through LDS; Y and D = T Y on VALU; then
// S <- exp(gC) S + K^T (F . D) on MFMA.
template <int DK, int DV, typename In>
__global__ __launch_bounds__(kThr) void cbwd_fwd(const In* __restrict__ k, const In* __restrict__ v,
                                                 const float* __restrict__ init, CWs w, int T, int H, int Hk,
                                                 int N, int vfirst) {
  constexpr int KP = DK + 4, MT = DK / 16, NT = (MT + 3) / 4, NW = MT < 4 ? MT : 4;
  __shared__ __align__(16) float kh[kC][KP];
  __shared__ float Tm[kC][kC + 1];
  __shared__ float part[NW][kC][kNS + 1];
  __shared__ float Y[kC][kNS + 1], FD[kC][kNS + 1];
  __shared__ TokVec tv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, li = lane & 15, lg = lane >> 4;
  constexpr int nsl = DV / kNS;
  const int sl = blockIdx.x % nsl, bh = blockIdx.x / nsl, b = bh / H, h = bh % H, hk = h / (H / Hk);
  const int n0 = sl * kNS;
  const long sb = static_cast<long>(bh) * DK * DV;
  auto sidx = [&](int c, int n) { return sb + (vfirst ? static_cast<long>(n) * DK + c : static_cast<long>(c) * DV + n); };
  f32x4 acc[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int mt = wave + 4 * j;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[j][e] = (mt < MT && init) ? init[sidx(16 * mt + 4 * lg + e, n0 + li)] : 0.f;
  }
  for (int ci = 0; ci < N; ++ci) {
    const int t0 = ci * kC, L = min(kC, T - t0);
    const long tok0 = static_cast<long>(b) * T + t0;
    float vv[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int idx = tid + u * kThr, r = idx / kNS, n = idx % kNS;
      vv[u] = r < L ? act<In>::load1(v + ((tok0 + r) * H + h) * DV + n0 + n) : 0.f;
    }
    __syncthreads();
    float* s0 = w.S0 + (static_cast<size_t>(bh) * N + ci) * DK * DV;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int mt = wave + 4 * j;
      if (mt < MT) {
#pragma unroll
        for (int e = 0; e < 4; ++e) s0[(16 * mt + 4 * lg + e) * DV + n0 + li] = acc[j][e];
      }
    }
    stage_rows<DK, KP, In>(kh, k, w.sk, tok0, H, h, Hk, hk, L, tid, kThr);
    stage_mats(Tm, nullptr, w, (static_cast<size_t>(bh) * N + ci) * kC * kC, tid, kThr);
    load_tokvec(tv, w, tok0, H, h, L, tid);
    __syncthreads();
    // K S over this wave's key rows: rows 16 rt + l % 16 of K, keys 16 mt + 4 (l / 16) + e
    if (wave < NW) {
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        f32x4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          const int mt = wave + 4 * j;
          if (mt < MT) {
            const f32x4 a = *reinterpret_cast<const f32x4*>(&kh[16 * rt + li][16 * mt + 4 * lg]);
#pragma unroll
            for (int e = 0; e < 4; ++e) p = mma4(a[e], acc[j][e], p);
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) part[wave][16 * rt + 4 * lg + e][li] = p[e];
      }
    }
    __syncthreads();
    // Y = beta . (V - exp(gx) . K S)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int idx = tid + u * kThr, r = idx / kNS, n = idx % kNS;
      float ks = 0.f;
#pragma unroll
      for (int q = 0; q < NW; ++q) ks += part[q][r][n];
      Y[r][n] = tv.bt[r] * (vv[u] - tv.egx[r] * ks);
    }
    __syncthreads();
    // F . D, D = T Y (T unit lower triangular)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int idx = tid + u * kThr, r = idx / kNS, n = idx % kNS;
      float d = 0.f;
      for (int s = 0; s <= r; ++s) d += Tm[r][s] * Y[s][n];
      FD[r][n] = tv.F[r] * d;
    }
    __syncthreads();
    // S <- exp(gC) S + K^T (F . D)
    const float egC = tv.egC;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int mt = wave + 4 * j;
      if (mt < MT) {
        acc[j] *= egC;
#pragma unroll
        for (int ks = 0; ks < kC / 4; ++ks) acc[j] = mma4(kh[4 * ks + lg][16 * mt + li], FD[4 * ks + lg][li], acc[j]);
      }
    }
  }
}

// (2) per (b, h, slice): the walk of the state gradient from the last chunk
// to the first; every chunk's dS1 into the workspace, dv, and the initial
// state's gradient.  The slice of dS sits in MFMA accumulators as S does in
// (1); per chunk: K dS (partial products per wave, summed through LDS),
// dD = P^T dO + F . K dS and dY = T^T dD on VALU, then
// dS <- exp(gC) dS + [Q; K]^T [exp(gam) . dO; -exp(gx) . dX] on MFMA.
template <int DK, int DV, typename In>
__global__ __launch_bounds__(kThr) void cbwd_rev(const In* __restrict__ q, const In* __restrict__ k,
                                                 const float* __restrict__ dout, const float* __restrict__ dfinal,
                                                 float* __restrict__ dv, float* __restrict__ dinit, CWs w, int T,
                                                 int H, int Hk, int N, int vfirst) {
  constexpr int KP = DK + 4, MT = DK / 16, NT = (MT + 3) / 4, NW = MT < 4 ? MT : 4;
  __shared__ __align__(16) float kh[kC][KP], qh[kC][KP];
  __shared__ float Tm[kC][kC + 1], Pm[kC][kC + 1];
  __shared__ float part[NW][kC][kNS + 1];
  __shared__ float dO[kC][kNS + 1], dD[kC][kNS + 1], BB[2 * kC][kNS + 1];
  __shared__ TokVec tv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, li = lane & 15, lg = lane >> 4;
  constexpr int nsl = DV / kNS;
  const int sl = blockIdx.x % nsl, bh = blockIdx.x / nsl, b = bh / H, h = bh % H, hk = h / (H / Hk);
  const int n0 = sl * kNS;
  const long sb = static_cast<long>(bh) * DK * DV;
  auto sidx = [&](int c, int n) { return sb + (vfirst ? static_cast<long>(n) * DK + c : static_cast<long>(c) * DV + n); };
  f32x4 acc[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int mt = wave + 4 * j;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[j][e] = (mt < MT && dfinal) ? dfinal[sidx(16 * mt + 4 * lg + e, n0 + li)] : 0.f;
  }
  for (int ci = N - 1; ci >= 0; --ci) {
    const int t0 = ci * kC, L = min(kC, T - t0);
    const long tok0 = static_cast<long>(b) * T + t0;
    float dov[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int idx = tid + u * kThr, r = idx / kNS, n = idx % kNS;
      dov[u] = r < L ? dout[((tok0 + r) * H + h) * DV + n0 + n] : 0.f;
    }
    __syncthreads();
    float* d1 = w.dS1 + (static_cast<size_t>(bh) * N + ci) * DK * DV;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int mt = wave + 4 * j;
      if (mt < MT) {
#pragma unroll
        for (int e = 0; e < 4; ++e) d1[(16 * mt + 4 * lg + e) * DV + n0 + li] = acc[j][e];
      }
    }
    stage_rows<DK, KP, In>(kh, k, w.sk, tok0, H, h, Hk, hk, L, tid, kThr);
    stage_rows<DK, KP, In>(qh, q, w.sq, tok0, H, h, Hk, hk, L, tid, kThr);
    stage_mats(Tm, Pm, w, (static_cast<size_t>(bh) * N + ci) * kC * kC, tid, kThr);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int idx = tid + u * kThr;
      dO[idx / kNS][idx % kNS] = dov[u];
    }
    load_tokvec(tv, w, tok0, H, h, L, tid);
    __syncthreads();
    // K dS over this wave's key rows
    if (wave < NW) {
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        f32x4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          const int mt = wave + 4 * j;
          if (mt < MT) {
            const f32x4 a = *reinterpret_cast<const f32x4*>(&kh[16 * rt + li][16 * mt + 4 * lg]);
#pragma unroll
            for (int e = 0; e < 4; ++e) p = mma4(a[e], acc[j][e], p);
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) part[wave][16 * rt + 4 * lg + e][li] = p[e];
      }
    }
    __syncthreads();
    // dD = P^T dO + F . K dS
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int idx = tid + u * kThr, r = idx / kNS, n = idx % kNS;
      float kd = 0.f;
#pragma unroll
      for (int qq = 0; qq < NW; ++qq) kd += part[qq][r][n];
      float pd = 0.f;
      for (int s = r; s < kC; ++s) pd += Pm[s][r] * dO[s][n];
      dD[r][n] = pd + tv.F[r] * kd;
    }
    __syncthreads();
    // dX = beta . T^T dD, the gradient of v; the B operand of the dS update
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int idx = tid + u * kThr, r = idx / kNS, n = idx % kNS;
      float y = 0.f;
      for (int s = r; s < kC; ++s) y += Tm[s][r] * dD[s][n];
      const float x = tv.bt[r] * y;
      if (r < L) dv[((tok0 + r) * H + h) * DV + n0 + n] = x;
      BB[r][n] = tv.egm[r] * dO[r][n];
      BB[kC + r][n] = -tv.egx[r] * x;
    }
    __syncthreads();
    // dS <- exp(gC) dS + Q^T (exp(gam) . dO) - K^T (exp(gx) . dX)
    const float egC = tv.egC;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int mt = wave + 4 * j;
      if (mt < MT) {
        acc[j] *= egC;
#pragma unroll
        for (int ks = 0; ks < kC / 4; ++ks) acc[j] = mma4(qh[4 * ks + lg][16 * mt + li], BB[4 * ks + lg][li], acc[j]);
#pragma unroll
        for (int ks = 0; ks < kC / 4; ++ks)
          acc[j] = mma4(kh[4 * ks + lg][16 * mt + li], BB[kC + 4 * ks + lg][li], acc[j]);
      }
    }
  }
  if (dinit) {
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int mt = wave + 4 * j;
      if (mt < MT) {
#pragma unroll
        for (int e = 0; e < 4; ++e) dinit[sidx(16 * mt + 4 * lg + e, n0 + li)] = acc[j][e];
      }
    }
  }
}

// (3) per (b, h, chunk): the remaining gradients over the value columns, 16
// at a time: dq and dk of the normalised rows (added: value heads of a group
// share their q/k head), dbeta and the decay's gradient (written).  Eight
// waves.  Per slice: [K S0 | Q S0 | K dS1] on MFMA (each wave a quarter of
// the keys of one row tile, summed through LDS); X, D, dD, dY and the
// per-token sums on VALU, one (row, column) element per thread; then on
// MFMA the running sums dT += dD Y^T, dP += dO D^T (a tile per wave) and
// dq += dO S0^T, dk += (F . D) dS1^T - (exp(gx) beta . dY) S0^T (tiles per
// wave, held across the slices).  Then dA, dG and Z on VALU and the last
// products dq += Z K, dk += (dG + dG^T) K + Z^T Q on MFMA.
template <int DK, int DV, typename In>
__global__ __launch_bounds__(kThr3) void cbwd_local(const In* __restrict__ q, const In* __restrict__ k,
                                                    const In* __restrict__ v, const float* __restrict__ dout,
                                                    float* __restrict__ dq, float* __restrict__ dk,
                                                    float* __restrict__ dbeta, float* __restrict__ ddecay,
                                                    CWs w, int T, int H, int Hk, int N) {
  constexpr int KP = DK + 4, NT16 = DK / 16, KQ = DK / 16;       // k-steps per quarter of the keys
  constexpr int NQK = 4 * NT16, TPW = (NQK + 7) / 8;              // dq/dk tiles, per wave
  constexpr int SPT = DK * kNS / kThr3;                          // state floats per thread per slice
  constexpr int SL = kNS / SPT;                                   // threads per state row
  constexpr int nsl = DV / kNS;
  __shared__ __align__(16) float kh[kC][KP], qh[kC][KP];
  __shared__ float S0s[DK][kNS + 1], S1s[DK][kNS + 1];
  __shared__ float part[4][3][kC][kNS + 1];
  __shared__ float Tm[kC][kC + 1], Pm[kC][kC + 1];
  __shared__ float dO[kC][kNS + 1], Yb[kC][kNS + 1], D[kC][kNS + 1], FD[kC][kNS + 1];
  __shared__ float dD[kC][kNS + 1], dYs[kC][kNS + 1];
  __shared__ float dTm[kC][kC + 1], dPm[kC][kC + 1], M[kC][kC + 1], EE[kC][kC + 1], PP[kC][kC + 1];
  __shared__ float Gp[2][kC][kC + 1], dGs[kC][kC + 1];
  __shared__ float tb[kC], tm[kC], tx[kC], tc[kC], sgm[kC], sgx[kC], red[8];
  __shared__ TokVec tv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, li = lane & 15, lg = lane >> 4;
  const int er = tid / kNS, en = tid % kNS;   // this thread's element of a 32 x 16 slice tile
  const int ci = blockIdx.x % N, bh = blockIdx.x / N, b = bh / H, h = bh % H, hk = h / (H / Hk);
  const int t0 = ci * kC, L = min(kC, T - t0);
  const long tok0 = static_cast<long>(b) * T + t0;
  const size_t cb = (static_cast<size_t>(bh) * N + ci) * kC * kC;
  const float* s0g = w.S0 + (static_cast<size_t>(bh) * N + ci) * DK * DV;
  const float* s1g = w.dS1 + (static_cast<size_t>(bh) * N + ci) * DK * DV;
  const bool rin = er < L;
  const long vrow = ((tok0 + er) * H + h) * DV;
  const int sc = tid / SL, sn = (tid % SL) * SPT;   // this thread's state elements: row sc, columns sn..
  float ps0[SPT], ps1[SPT], pdo, pv;
  auto prefetch = [&](int s) {
    const int nb = s * kNS;
#pragma unroll
    for (int e = 0; e < SPT; ++e) {
      ps0[e] = s0g[sc * DV + nb + sn + e];
      ps1[e] = s1g[sc * DV + nb + sn + e];
    }
    pdo = rin ? dout[vrow + nb + en] : 0.f;
    pv = rin ? act<In>::load1(v + vrow + nb + en) : 0.f;
  };
  prefetch(0);
  stage_rows<DK, KP, In>(kh, k, w.sk, tok0, H, h, Hk, hk, L, tid, kThr3);
  stage_rows<DK, KP, In>(qh, q, w.sq, tok0, H, h, Hk, hk, L, tid, kThr3);
  stage_mats(Tm, Pm, w, cb, tid, kThr3);
  load_tokvec(tv, w, tok0, H, h, L, tid);
  if (tid < kC) {
    sgm[tid] = tid < L ? w.gm[(tok0 + tid) * H + h] : 0.f;
    sgx[tid] = tid < L ? w.gx[(tok0 + tid) * H + h] : 0.f;
  }
  float sb = 0.f, so = 0.f, sx = 0.f, sf = 0.f, sdc = 0.f;   // per-token sums (this thread's columns)
  f32x4 atp = {0.f, 0.f, 0.f, 0.f};                          // dT (waves 0-3) or dP (4-7) tile
  f32x4 aqk[TPW];
#pragma unroll
  for (int j = 0; j < TPW; ++j) aqk[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int tpm = wave >> 2, tpr = (wave >> 1) & 1, tpc = wave & 1;
  const int pmt = wave & 1, pq = wave >> 1;                  // K-S product: row tile, key quarter
  for (int s = 0; s < nsl; ++s) {
    __syncthreads();
#pragma unroll
    for (int e = 0; e < SPT; ++e) {
      S0s[sc][sn + e] = ps0[e];
      S1s[sc][sn + e] = ps1[e];
      sdc += ps0[e] * ps1[e];
    }
    dO[er][en] = pdo;
    const float vcur = pv, docur = pdo;
    __syncthreads();
    if (s + 1 < nsl) prefetch(s + 1);
    // [K S0 | Q S0 | K dS1], this wave's row tile and key quarter
    {
      f32x4 p0 = {0.f, 0.f, 0.f, 0.f}, p1 = p0, p2 = p0;
#pragma unroll
      for (int ks = pq * KQ; ks < (pq + 1) * KQ; ++ks) {
        const float ak = kh[16 * pmt + li][4 * ks + lg], aq = qh[16 * pmt + li][4 * ks + lg];
        const float b0 = S0s[4 * ks + lg][li], b1 = S1s[4 * ks + lg][li];
        p0 = mma4(ak, b0, p0);
        p1 = mma4(aq, b0, p1);
        p2 = mma4(ak, b1, p2);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        part[pq][0][16 * pmt + 4 * lg + e][li] = p0[e];
        part[pq][1][16 * pmt + 4 * lg + e][li] = p1[e];
        part[pq][2][16 * pmt + 4 * lg + e][li] = p2[e];
      }
    }
    __syncthreads();
    float ksv = 0.f, qsv = 0.f, kdv = 0.f;
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      ksv += part[qq][0][er][en];
      qsv += part[qq][1][er][en];
      kdv += part[qq][2][er][en];
    }
    const float x = vcur - tv.egx[er] * ksv;
    Yb[er][en] = tv.bt[er] * x;
    __syncthreads();
    // D = T Y;  dD = P^T dO + F . K dS1
    float d = 0.f, pd = 0.f;
    for (int t = 0; t <= er; ++t) d += Tm[er][t] * Yb[t][en];
    for (int t = er; t < kC; ++t) pd += Pm[t][er] * dO[t][en];
    const float dd = pd + tv.F[er] * kdv;
    D[er][en] = d;
    FD[er][en] = tv.F[er] * d;
    dD[er][en] = dd;
    __syncthreads();
    // dY = T^T dD, and the per-token sums
    float y = 0.f;
    for (int t = er; t < kC; ++t) y += Tm[t][er] * dD[t][en];
    dYs[er][en] = -tv.egx[er] * tv.bt[er] * y;
    sb += y * x;
    so += docur * qsv;
    sx += y * (vcur - x);
    sf += kdv * d;
    __syncthreads();
    // dT += dD Y^T, dP += dO D^T (this wave's tile)
#pragma unroll
    for (int ks = 0; ks < kNS / 4; ++ks) {
      const float a = tpm ? dO[16 * tpr + li][4 * ks + lg] : dD[16 * tpr + li][4 * ks + lg];
      const float bb = tpm ? D[16 * tpc + li][4 * ks + lg] : Yb[16 * tpc + li][4 * ks + lg];
      atp = mma4(a, bb, atp);
    }
    // dq += dO S0^T;  dk += (F . D) dS1^T + (-exp(gx) beta . dY) S0^T
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      const int t = wave + 8 * j;
      if (t < NQK) {
        const int mat = t / (2 * NT16), rem = t % (2 * NT16), mt = rem / NT16, nt = rem % NT16;
#pragma unroll
        for (int ks = 0; ks < kNS / 4; ++ks) {
          const int r = 16 * mt + li, n = 4 * ks + lg, c = 16 * nt + li;
          if (mat == 0) {
            aqk[j] = mma4(dO[r][n], S0s[c][n], aqk[j]);
          } else {
            aqk[j] = mma4(FD[r][n], S1s[c][n], aqk[j]);
            aqk[j] = mma4(dYs[r][n], S0s[c][n], aqk[j]);
          }
        }
      }
    }
  }
  // per-token sums over the 16 columns of a row (16 consecutive lanes)
  sb = dpp_group_sum<16>(sb);
  so = dpp_group_sum<16>(so);
  sx = dpp_group_sum<16>(sx);
  sf = dpp_group_sum<16>(sf);
  sdc = dpp_group_sum<64>(sdc);
  __syncthreads();
  if (en == 0) {
    tb[er] = sb;
    tm[er] = tv.egm[er] * so - tv.F[er] * sf;
    tx[er] = -tv.bt[er] * sx;
    tc[er] = tv.F[er] * sf;
  }
  if (lane == 0) red[wave] = sdc;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int r = 16 * tpr + 4 * lg + e, c = 16 * tpc + li;
    if (tpm) dPm[r][c] = atp[e];
    else dTm[r][c] = c <= r ? atp[e] : 0.f;
  }
  __syncthreads();
  // M = dT T^T (dT, T lower): M_rs = sum_{u <= min(r, s)} dT_ru T_su; K K^T on MFMA
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int idx = tid + u * kThr3, r = idx / kC, c = idx % kC, um = min(r, c);
    float m = 0.f;
    for (int t = 0; t <= um; ++t) m += dTm[r][t] * Tm[c][t];
    M[r][c] = m;
  }
  {
    const int gt = wave & 3, gr = gt >> 1, gc = gt & 1, gh = wave >> 2;
    f32x4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = gh * (DK / 8); ks < (gh + 1) * (DK / 8); ++ks)
      p = mma4(kh[16 * gr + li][4 * ks + lg], kh[16 * gc + li][4 * ks + lg], p);
#pragma unroll
    for (int e = 0; e < 4; ++e) Gp[gh][16 * gr + 4 * lg + e][16 * gc + li] = p[e];
  }
  __syncthreads();
  // dA = -T^T M on s < r; E = dA . (K K^T) . W; dG = diag(beta) dA . W;
  // Z = dP . Vw (into dPm) and dP . P
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int idx = tid + u * kThr3, r = idx / kC, c = idx % kC;
    float e = 0.f, dg = 0.f;
    if (c < r) {
      float da = 0.f;
      for (int t = r; t < kC; ++t) da -= Tm[t][r] * M[t][c];
      const float wr = __expf(sgx[r] - sgm[c]);
      e = da * (Gp[0][r][c] + Gp[1][r][c]) * wr;
      dg = da * tv.bt[r] * wr;
    }
    EE[r][c] = e;
    Gp[0][r][c] = dg;   // this thread's own element of Gp, read above: dG in its place
    const float dp = c <= r ? dPm[r][c] : 0.f;
    PP[r][c] = dp * Pm[r][c];
    dPm[r][c] = c <= r ? dp * __expf(sgm[r] - sgm[c]) : 0.f;
  }
  __syncthreads();
  if (tid < kC) {
    const int r = tid;
    float re = 0.f, rp = 0.f, ce = 0.f, cp = 0.f;
    for (int t = 0; t < kC; ++t) {
      re += EE[r][t];
      rp += PP[r][t];
      ce += tv.bt[t] * EE[t][r];
      cp += PP[t][r];
    }
    tb[r] += re;
    tx[r] += tv.bt[r] * re;
    tm[r] += rp - ce - cp;
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int idx = tid + u * kThr3, r = idx / kC, c = idx % kC;
    dGs[r][c] = Gp[0][r][c] + Gp[0][c][r];
  }
  __syncthreads();
  // dq = exp(gam) . (dO S0^T) + Z K;  dk += (dG + dG^T) K + Z^T Q; into the outputs
  const bool grouped = H != Hk;
#pragma unroll
  for (int j = 0; j < TPW; ++j) {
    const int t = wave + 8 * j;
    if (t < NQK) {
      const int mat = t / (2 * NT16), rem = t % (2 * NT16), mt = rem / NT16, nt = rem % NT16;
      f32x4 a = aqk[j];
      if (mat == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) a[e] *= tv.egm[16 * mt + 4 * lg + e];
#pragma unroll
        for (int ks = 0; ks < kC / 4; ++ks) a = mma4(dPm[16 * mt + li][4 * ks + lg], kh[4 * ks + lg][16 * nt + li], a);
      } else {
#pragma unroll
        for (int ks = 0; ks < kC / 4; ++ks) {
          a = mma4(dGs[16 * mt + li][4 * ks + lg], kh[4 * ks + lg][16 * nt + li], a);
          a = mma4(dPm[4 * ks + lg][16 * mt + li], qh[4 * ks + lg][16 * nt + li], a);
        }
      }
      float* out = mat == 0 ? dq : dk;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * mt + 4 * lg + e;
        if (r < L) {
          const long o = ((tok0 + r) * Hk + hk) * DK + 16 * nt + li;
          if (grouped) atomicAdd(out + o, a[e]);
          else out[o] = a[e];
        }
      }
    }
  }
  // dg_t = sum_{r >= t} dgam_r + sum_{r > t} dgx_r + dgC
  if (tid < kC) {
    const int t = tid;
    if (t < L) {
      float dgc = 0.f, sg = 0.f;
#pragma unroll
      for (int wv = 0; wv < 8; ++wv) dgc += red[wv];
      dgc *= tv.egC;
      for (int r = 0; r < kC; ++r) {
        dgc += tc[r];
        if (r >= t) sg += tm[r];
        if (r > t) sg += tx[r];
      }
      const long ti = (tok0 + t) * H + h;
      dbeta[ti] = tb[t];
      if (ddecay) ddecay[ti] = sg + dgc;
    }
  }
}

template <int DK, int DV, typename In>
hipError_t run(const BwdArgs& a, hipStream_t s) {
  const In* q = static_cast<const In*>(a.q);
  const In* k = static_cast<const In*>(a.k);
  const In* v = static_cast<const In*>(a.v);
  const In* be = static_cast<const In*>(a.beta);
  const In* de = static_cast<const In*>(a.decay);
  const int N = (a.T + kC - 1) / kC;
  CWs w;
  ws_floats(a.B, a.T, a.H, DK, DV, &w, a.ckpt);
  const unsigned chunks = static_cast<unsigned>(a.B * a.H * N), slices = static_cast<unsigned>(a.B * a.H * (DV / kNS));
  cbwd_prep<DK, In><<<dim3(chunks), dim3(kThr), 0, s>>>(q, k, be, de, a.decay_kind == DECAY_HEAD, w, a.T, a.H,
                                                         a.Hk, N, a.scale, a.l2norm, a.tf);
  cbwd_fwd<DK, DV, In><<<dim3(slices), dim3(kThr), 0, s>>>(k, v, a.init, w, a.T, a.H, a.Hk, N, a.vfirst);
  cbwd_rev<DK, DV, In><<<dim3(slices), dim3(kThr), 0, s>>>(q, k, a.dout, a.dfinal, a.dv, a.dinit, w, a.T, a.H,
                                                           a.Hk, N, a.vfirst);
  cbwd_local<DK, DV, In><<<dim3(chunks), dim3(kThr3), 0, s>>>(
      q, k, v, a.dout, a.dq, a.dk, a.dbeta, a.decay_kind == DECAY_HEAD ? a.ddecay : nullptr, w, a.T, a.H, a.Hk, N);
  return hipGetLastError();
}

template <typename In>
hipError_t dispatch(const BwdArgs& a, hipStream_t s) {
#define KDA_CBWD_CASE(dk_, dv_) \
  if (a.DK == dk_ && a.DV == dv_) return run<dk_, dv_, In>(a, s);
  KDA_CBWD_CASE(32, 32) KDA_CBWD_CASE(32, 64) KDA_CBWD_CASE(32, 128)
  KDA_CBWD_CASE(64, 32) KDA_CBWD_CASE(64, 64) KDA_CBWD_CASE(64, 128)
  KDA_CBWD_CASE(128, 32) KDA_CBWD_CASE(128, 64) KDA_CBWD_CASE(128, 128)
#undef KDA_CBWD_CASE
  return hipErrorInvalidValue;
}

}  // namespace

size_t bwd_chunked_workspace_bytes(int B, int T, int H, int DK, int DV) {
  return ws_floats(B, T, H, DK, DV, nullptr, nullptr) * sizeof(float);
}

hipError_t launch_bwd_chunked(const BwdArgs& a, hipStream_t s) {
  return a.dtype == 0 ? dispatch<float>(a, s) : dispatch<bf16_t>(a, s);
}

}  // namespace kda
