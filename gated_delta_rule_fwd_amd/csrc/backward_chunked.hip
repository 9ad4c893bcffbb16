// Chunked backward of the gated delta rule: the gradients of (o, final state)
// with respect to q, k, v, beta, the decay and the initial state, computed
// chunk by chunk in the WY form that the forward uses (TileOPs "Linear
// Attention Operators": the DeltaNet chunked pipeline and its
// DeltaNetChunkBwdOp, GLAChunkBwdOp for the decay; kda-neuron-kernels README,
// kda_chunk_step_exact_bwd).
//
// For a chunk of C tokens entering with state S0, with q, k the normalised
// (q scaled) rows, gam the inclusive and gx the exclusive in-chunk cumulative
// log decay, gC the chunk's total and F = exp(gC - gam), with a per-head
// decay (none: all zero):
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
// With a per-channel decay the same holds with every decay factor taken per
// key channel c: exp(gx_rc), exp(gam_rc) and exp(gC_c - gam_rc) scale k and q
// channel by channel, exp(gC_c) scales state row c, and an entry of A or P
// sums over the channels with its own factor exp(gx_rc - gam_sc) or
// exp(gam_rc - gam_sc); the gradients of those pair terms, and of the decay,
// are taken per (token, channel).
//
// Four kernels: (0) per chunk, in parallel: the rows' norm factors, beta,
// the cumulative decays, T and P; (1) per (b, h, kNS value columns): the
// walk over the chunks storing each chunk's S0; (2) the same slices in
// reverse: the walk of the state gradient storing each chunk's dS1 and
// writing dv and the initial state's gradient (2 kNS columns per workgroup
// when slices of kNS would exceed two per CU); (3) per chunk, in parallel:
// everything else, over the value columns kNS at a time.  (0) and (3) have a
// per-channel version each; (1) and (2) a per-channel mode.  (3) also
// carries dq and dk through the L2 norm and the scale when every q/k head has
// one value head; with grouped heads it adds the normalised rows' gradients
// over the group and a last kernel (backward.hip) takes the norm.  All
// arithmetic is fp32.
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
  float* gmc;                      // [B*T*H][DK]: gam per key channel (per-channel decay)
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
    w->dS1 = p; p += st;
    w->gmc = p;
  }
  return 5 * tok + 2 * mats + 2 * st + static_cast<size_t>(B) * T * H * DK;
}

// Workgroup barrier ordering LDS accesses only: global loads in flight (the
// next chunk's or slice's operands) are not waited for, as __syncthreads
// would.
__device__ __forceinline__ void lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// acc += A (16 x 4) B (4 x 16), fp32: lane l gives A[l % 16][l / 16] and
// B[l / 16][l % 16]; it holds rows 4 (l / 16) + j, j = 0..3, of column l % 16.
__device__ __forceinline__ f32x4 mma4(float a, float b, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
}

// LDS pitch of 32 x 32 matrices: rows read as 16-byte vectors
constexpr int kCP = kC + 4;

// (0) per (b, h, chunk): the norm factors of the rows, beta and the
// cumulative decays per token; T and P of the chunk.
// Column j of T = (I + A)^-1 (A strictly lower, kC x kC in LDS) by forward
// substitution, each row's sum in four partial sums (a chain a quarter as
// long).  A's rows are read four entries at a time, row r + 1 while row r
// is summed (the scheduling fence keeps those reads ahead of the sums).
__device__ __forceinline__ void tri_inv_col(const float (*sA)[kCP], int j, float (&x)[kC]) {
  x[0] = j == 0 ? 1.f : 0.f;
  f32x4 cur[kC / 4], nxt[kC / 4];
  cur[0] = *reinterpret_cast<const f32x4*>(&sA[1][0]);
#pragma unroll
  for (int r = 1; r < kC; ++r) {
    if (r + 1 < kC) {
#pragma unroll
      for (int s4 = 0; s4 < (r + 4) / 4; ++s4) nxt[s4] = *reinterpret_cast<const f32x4*>(&sA[r + 1][4 * s4]);
    }
    __builtin_amdgcn_sched_barrier(0);
    float a[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s4 = 0; s4 < (r + 3) / 4; ++s4) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (4 * s4 + e < r) a[e] += cur[s4][e] * x[4 * s4 + e];
    }
    x[r] = (r == j ? 1.f : 0.f) - ((a[0] + a[1]) + (a[2] + a[3]));
#pragma unroll
    for (int s4 = 0; s4 < kC / 4; ++s4) cur[s4] = nxt[s4];
  }
}

template <int DK, typename In>
__global__ __launch_bounds__(kThr) void cbwd_prep(const In* __restrict__ q, const In* __restrict__ k,
                                                  const In* __restrict__ beta, const In* __restrict__ decay,
                                                  int headd, CWs w, int T, int H, int Hk, int N, float scale,
                                                  int l2norm, Transforms tf) {
  constexpr int KP = DK + 4;
  __shared__ __align__(16) float kh[kC][KP], qh[kC][KP];
  __shared__ __align__(16) float sA[kC][kCP];
  __shared__ float sbt[kC], sgm[kC], sgx[kC];
  const int tid = threadIdx.x;
  const int ci = blockIdx.x % N, bh = blockIdx.x / N, b = bh / H, h = bh % H, hk = h / (H / Hk);
  const int t0 = ci * kC, L = min(kC, T - t0);
  const long tok0 = static_cast<long>(b) * T + t0;
  {
    // LPR lanes to a row, one 16-byte load of q and of k each
    constexpr int V = act<In>::kVec, LPR = DK / V;
    static_assert(kC * LPR % 64 == 0, "whole waves per pass");
    for (int idx = tid; idx < kC * LPR; idx += kThr) {
      const int r = idx / LPR, seg = idx % LPR;
      const bool in = r < L;
      float qv[V], kv[V], sq = 0.f, sk = 0.f;
      if (in) {
        const long base = ((tok0 + r) * Hk + hk) * DK + seg * V;
        act<In>::load_vec(q + base, qv);
        act<In>::load_vec(k + base, kv);
      } else {
#pragma unroll
        for (int e = 0; e < V; ++e) qv[e] = kv[e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < V; ++e) {
        sq += qv[e] * qv[e];
        sk += kv[e] * kv[e];
      }
      sq = dpp_group_sum<LPR>(sq);
      sk = dpp_group_sum<LPR>(sk);
      const float fq = (l2norm ? inv_norm(sq) : 1.f) * scale, fk = l2norm ? inv_norm(sk) : 1.f;
#pragma unroll
      for (int e = 0; e < V; ++e) {
        qh[r][seg * V + e] = qv[e] * fq;
        kh[r][seg * V + e] = kv[e] * fk;
      }
      if (seg == 0 && in) {
        w.sq[(tok0 + r) * H + h] = fq;
        w.sk[(tok0 + r) * H + h] = fk;
      }
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
  lds_sync();
  const size_t cb = (static_cast<size_t>(bh) * N + ci) * kC * kC;
  {
    // K K^T and Q K^T on MFMA, a 16 x 16 tile of each per wave (the upper
    // tile is zero); a 16-byte row read feeds four products, k = 4 (l / 16) + e
    const int wave = tid >> 6, lane = tid & 63, li = lane & 15, lg = lane >> 4;
    const int rt = wave >> 1, ct = wave & 1;
    f32x4 g = {0.f, 0.f, 0.f, 0.f}, p = g;
    if (ct <= rt) {
#pragma unroll 4
      for (int kb = 0; kb < DK / 16; ++kb) {
        const f32x4 ak = *reinterpret_cast<const f32x4*>(&kh[16 * rt + li][16 * kb + 4 * lg]);
        const f32x4 aq = *reinterpret_cast<const f32x4*>(&qh[16 * rt + li][16 * kb + 4 * lg]);
        const f32x4 bk = *reinterpret_cast<const f32x4*>(&kh[16 * ct + li][16 * kb + 4 * lg]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          g = mma4(ak[e], bk[e], g);
          p = mma4(aq[e], bk[e], p);
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 * rt + 4 * lg + e, s = 16 * ct + li;
      sA[r][s] = s < r ? sbt[r] * g[e] * __expf(sgx[r] - sgm[s]) : 0.f;
      w.Pm[cb + r * kC + s] = s <= r ? p[e] * __expf(sgm[r] - sgm[s]) : 0.f;
    }
  }
  lds_sync();
  if (tid < kC) {
    // column j of T = (I + A)^-1
    const int j = tid;
    float x[kC];
    tri_inv_col(sA, j, x);
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
// One chunk's token values, loaded ahead (lanes 0..31 of wave 0 use them).
// Loads here and below are unconditional, from clamped in-range addresses,
// and the values are masked when stored: nothing waits on a load before its
// values are stored to LDS.
struct TokPf {
  float bt, gx, gm, gC;
  __device__ void load(const CWs& w, long tok0, int H, int h, int L, int tid) {
    const long t = (tok0 + min(tid & (kC - 1), L - 1)) * H + h;
    bt = w.bt[t];
    gx = w.gx[t];
    gm = w.gm[t];
    gC = w.gm[(tok0 + L - 1) * H + h];
  }
  // CH (per-channel decay): the decay factors are per key channel and
  // applied elsewhere; the per-token ones are left at one
  template <bool CH = false>
  __device__ void store(TokVec& tv, int L, int tid) const {
    if (tid < kC) {
      const bool in = tid < L;
      tv.bt[tid] = in ? bt : 0.f;
      tv.egx[tid] = in ? (CH ? 1.f : __expf(gx)) : 0.f;
      tv.egm[tid] = in ? (CH ? 1.f : __expf(gm)) : 0.f;
      tv.F[tid] = in ? (CH ? 1.f : __expf(gC - gm)) : 0.f;
      if (tid == 0) tv.egC = CH ? 1.f : __expf(gC);
    }
  }
};

// One chunk's cumulative decay per key channel (gam, fp32), loaded ahead;
// stored as rows 1..32 of an LDS array whose row 0 is zero, so that row r
// holds gx and row r + 1 gam of token r (rows past the end repeat the last
// token's, which is gC).
template <int DK, int NTHR>
struct GamPf {
  static constexpr int NV = kC * DK / 4, NPT = (NV + NTHR - 1) / NTHR;
  f32x4 g[NPT];
  __device__ void load(const float* gmc, long tok0, int H, int h, int L, int tid) {
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      const int idx = min(tid + i * NTHR, NV - 1), r = min(idx / (DK / 4), L - 1), c4 = (idx % (DK / 4)) * 4;
      g[i] = *reinterpret_cast<const f32x4*>(gmc + ((tok0 + r) * H + h) * DK + c4);
    }
  }
  template <int KP>
  __device__ void store(float (*gs)[KP], int tid) const {
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      const int idx = tid + i * NTHR, r = idx / (DK / 4), c4 = (idx % (DK / 4)) * 4;
      if (idx < NV) *reinterpret_cast<f32x4*>(&gs[r + 1][c4]) = g[i];
    }
  }
};

// Raw 16-byte vectors and single elements of the input type, converted to
// fp32 only when used
template <typename In> struct Raw;
template <> struct Raw<float> {
  using vec = f32x4;
  using one = float;
  static constexpr int V = 4;
  __device__ static void cvt(const vec& r, float (&o)[4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = r[e];
  }
  __device__ static one ld1(const float* p) { return *p; }
  __device__ static float cvt1(one x) { return x; }
};
template <> struct Raw<bf16_t> {
  using vec = uint4;
  using one = uint16_t;
  static constexpr int V = 8;
  __device__ static void cvt(const vec& r, float (&o)[8]) {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = __uint_as_float(w[i] << 16);
      o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ static one ld1(const bf16_t* p) { return p->bits; }
  __device__ static float cvt1(one x) { return bf16_to_f32(x); }
};

// The raw rows of a chunk and their norm factors, loaded ahead into
// registers (NTHR threads, one 16-byte load per pass); store() writes the
// normalised rows into LDS rows of pitch KP (rows past the end: zeros).
template <int DK, typename In, int NTHR>
struct RowPf {
  static constexpr int V = Raw<In>::V, LPR = DK / V, NPT = (kC * LPR + NTHR - 1) / NTHR;
  typename Raw<In>::vec x[NPT];
  float f[NPT];
  __device__ void load(const In* src, const float* fac, long tok0, int H, int h, int Hk, int hk, int L, int tid) {
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      const int idx = min(tid + i * NTHR, kC * LPR - 1), r = min(idx / LPR, L - 1), seg = idx % LPR;
      x[i] = *reinterpret_cast<const typename Raw<In>::vec*>(src + ((tok0 + r) * Hk + hk) * DK + seg * V);
      f[i] = fac[(tok0 + r) * H + h];
    }
  }
  template <int KP>
  __device__ void store(float (*dst)[KP], int L, int tid) const {
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      const int idx = tid + i * NTHR, r = idx / LPR, seg = idx % LPR;
      if (idx < kC * LPR) {
        float v[V];
        Raw<In>::cvt(x[i], v);
        const float fr = r < L ? f[i] : 0.f;
#pragma unroll
        for (int e = 0; e < V; ++e) dst[r][seg * V + e] = r < L ? v[e] * fr : 0.f;
      }
    }
  }
};

// T and P of a chunk, loaded ahead (NTHR threads, 16-byte loads); stored
// into LDS transposed (T^T, P^T) and, if given, as they are
template <int NTHR, bool withP>
struct MatPf {
  static constexpr int NPT = (kC * kC / 4 + NTHR - 1) / NTHR;
  f32x4 t[NPT], p[NPT];
  __device__ void load(const CWs& w, size_t cb, int tid) {
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      const int idx = min(tid + i * NTHR, kC * kC / 4 - 1);
      t[i] = *reinterpret_cast<const f32x4*>(w.Tm + cb + 4 * idx);
      if (withP) p[i] = *reinterpret_cast<const f32x4*>(w.Pm + cb + 4 * idx);
    }
  }
  __device__ void store(float (*Td)[kCP], float (*TdT)[kCP], float (*PdT)[kCP], int tid) const {
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      const int idx = tid + i * NTHR, r = idx / (kC / 4), c4 = (idx % (kC / 4)) * 4;
      if (idx < kC * kC / 4) {
        if (Td) *reinterpret_cast<f32x4*>(&Td[r][c4]) = t[i];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (TdT) TdT[c4 + e][r] = t[i][e];
          if (withP && PdT) PdT[c4 + e][r] = p[i][e];
        }
      }
    }
  }
};

// The 16 x 16 tile (rt, ct) of two 32 x 32 products on fp32 MFMA, with T
// given transposed (TmT[t][r] = T_rt): M = dT T^T, dT and T both lower
// triangular (tokens t <= min(r, c) only), and T^T M (tokens t >= r only).
__device__ __forceinline__ f32x4 tile_dt_tt(const float (*dTm)[kCP], const float (*TmT)[kCP], int rt, int ct,
                                            int li, int lg) {
  f32x4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < kC / 16; ++kb) {
    if (kb <= rt && kb <= ct) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(&dTm[16 * rt + li][16 * kb + 4 * lg]);
#pragma unroll
      for (int e = 0; e < 4; ++e) p = mma4(a[e], TmT[16 * kb + 4 * lg + e][16 * ct + li], p);
    }
  }
  return p;
}
__device__ __forceinline__ f32x4 tile_tt_m(const float (*TmT)[kCP], const float (*Mm)[kCP], int rt, int ct,
                                           int li, int lg) {
  f32x4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < kC / 16; ++kb) {
    if (kb >= rt) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(&TmT[16 * rt + li][16 * kb + 4 * lg]);
#pragma unroll
      for (int e = 0; e < 4; ++e) p = mma4(a[e], Mm[16 * kb + 4 * lg + e][16 * ct + li], p);
    }
  }
  return p;
}

// (1) per (b, h, slice of kNS value columns): every chunk's S0 into the
// workspace, chunk after chunk.  The slice of the state (DK x 16) sits in
// MFMA accumulators, 16 key rows per tile, tile m in wave m % 4.  Per chunk:
// K S as partial products of each wave's own tiles (the tile is the B
// operand as it stands), summed through LDS; Y on VALU; D = T Y and then
// S <- exp(gC) S + K^T (F . D) on MFMA.  The next chunk's inputs are loaded
// into registers while this one is computed.
template <int DK, int DV, typename In, bool CH>
__global__ __launch_bounds__(kThr) void cbwd_fwd(const In* __restrict__ k, const In* __restrict__ v,
                                                 const float* __restrict__ init, CWs w, int T, int H, int Hk,
                                                 int N, int vfirst) {
  constexpr int KP = DK + 4, MT = DK / 16, NT = (MT + 3) / 4, NW = MT < 4 ? MT : 4;
  __shared__ __align__(16) float kh[kC][KP];
  // per-channel decay: gam per key channel, row r + 1 for token r (row 0: zeros)
  __shared__ __align__(16) float gs[CH ? kC + 1 : 1][CH ? KP : 4];
  __shared__ __align__(16) float Tm[kC][kCP];
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
  RowPf<DK, In, kThr> kpf;
  MatPf<kThr, false> mpf;
  TokPf tpf;
  GamPf<CH ? DK : 4, kThr> gpf;
  if (CH)
    for (int c = tid; c < DK; c += kThr) gs[0][c] = 0.f;
  typename Raw<In>::one vv[2];
  auto prefetch = [&](int c) __attribute__((always_inline)) {
    const int L = min(kC, T - c * kC);
    const long tok0 = static_cast<long>(b) * T + c * kC;
    kpf.load(k, w.sk, tok0, H, h, Hk, hk, L, tid);
    mpf.load(w, (static_cast<size_t>(bh) * N + c) * kC * kC, tid);
    tpf.load(w, tok0, H, h, L, tid);
    if constexpr (CH) gpf.load(w.gmc, tok0, H, h, L, tid);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int idx = tid + u * kThr, r = min(idx / kNS, L - 1), n = idx % kNS;
      vv[u] = Raw<In>::ld1(v + ((tok0 + r) * H + h) * DV + n0 + n);
    }
  };
  prefetch(0);
  for (int ci = 0; ci < N; ++ci) {
    const int L = min(kC, T - ci * kC);
    lds_sync();
    kpf.store(kh, L, tid);
    mpf.store(Tm, nullptr, nullptr, tid);
    tpf.store<CH>(tv, L, tid);
    if constexpr (CH) gpf.store(gs, tid);
    const float v0 = (tid / kNS) < L ? Raw<In>::cvt1(vv[0]) : 0.f;
    const float v1 = (tid + kThr) / kNS < L ? Raw<In>::cvt1(vv[1]) : 0.f;
    float* s0 = w.S0 + (static_cast<size_t>(bh) * N + ci) * DK * DV;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int mt = wave + 4 * j;
      if (mt < MT) {
#pragma unroll
        for (int e = 0; e < 4; ++e) s0[(16 * mt + 4 * lg + e) * DV + n0 + li] = acc[j][e];
      }
    }
    lds_sync();
    if (ci + 1 < N) prefetch(ci + 1);
    // K S over this wave's key rows: rows 16 rt + l % 16 of K, keys 16 mt + 4 (l / 16) + e
    if (wave < NW) {
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        f32x4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          const int mt = wave + 4 * j;
          if (mt < MT) {
            f32x4 a = *reinterpret_cast<const f32x4*>(&kh[16 * rt + li][16 * mt + 4 * lg]);
            if constexpr (CH) {
              // k exp(gx) per channel
              const f32x4 gx = *reinterpret_cast<const f32x4*>(&gs[16 * rt + li][16 * mt + 4 * lg]);
#pragma unroll
              for (int e = 0; e < 4; ++e) a[e] *= __expf(gx[e]);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) p = mma4(a[e], acc[j][e], p);
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) part[wave][16 * rt + 4 * lg + e][li] = p[e];
      }
    }
    lds_sync();
    // Y = beta . (V - exp(gx) . K S)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int idx = tid + u * kThr, r = idx / kNS, n = idx % kNS;
      float ks = 0.f;
#pragma unroll
      for (int q = 0; q < NW; ++q) ks += part[q][r][n];
      Y[r][n] = tv.bt[r] * ((u ? v1 : v0) - tv.egx[r] * ks);
    }
    lds_sync();
    // F . D, D = T Y on MFMA (waves 0, 1, a row tile each; T is unit lower
    // triangular, so row tile 0 takes tokens 0..15 only)
    if (wave < 2) {
      f32x4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < kC / 16; ++kb) {
        if (kb <= wave) {
          const f32x4 a = *reinterpret_cast<const f32x4*>(&Tm[16 * wave + li][16 * kb + 4 * lg]);
#pragma unroll
          for (int e = 0; e < 4; ++e) p = mma4(a[e], Y[16 * kb + 4 * lg + e][li], p);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * wave + 4 * lg + e;
        FD[r][li] = tv.F[r] * p[e];
      }
    }
    lds_sync();
    // S <- exp(gC) S + K^T (F . D); per channel: exp(gC_c) per state row and
    // F = exp(gC_c - gam_rc) in the K operand
    const float egC = tv.egC;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int mt = wave + 4 * j;
      if (mt < MT) {
        if constexpr (CH) {
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[j][e] *= __expf(gs[L][16 * mt + 4 * lg + e]);
          const float gC = gs[L][16 * mt + li];
#pragma unroll
          for (int ks = 0; ks < kC / 4; ++ks) {
            const int r = 4 * ks + lg;
            acc[j] = mma4(kh[r][16 * mt + li] * __expf(gC - gs[r + 1][16 * mt + li]), FD[r][li], acc[j]);
          }
        } else {
          acc[j] *= egC;
#pragma unroll
          for (int ks = 0; ks < kC / 4; ++ks) acc[j] = mma4(kh[4 * ks + lg][16 * mt + li], FD[4 * ks + lg][li], acc[j]);
        }
      }
    }
  }
}

// (2) per (b, h, slice): the walk of the state gradient from the last chunk
// to the first; every chunk's dS1 into the workspace, dv, and the initial
// state's gradient.  The slice of dS sits in MFMA accumulators as S does in
// (1); per chunk: K dS (partial products per wave, summed through LDS) and
// P^T dO on MFMA, dD = P^T dO + F . K dS on VALU, dY = T^T dD on MFMA, then
// dS <- exp(gC) dS + [Q; K]^T [exp(gam) . dO; -exp(gx) . dX] on MFMA.  The
// next chunk's inputs are loaded into registers while this one is computed.
template <int DK, int DV, typename In, bool CH, int NS>
__global__ __launch_bounds__(kThr) void cbwd_rev(const In* __restrict__ q, const In* __restrict__ k,
                                                 const float* __restrict__ dout, const float* __restrict__ dfinal,
                                                 float* __restrict__ dv, float* __restrict__ dinit, CWs w, int T,
                                                 int H, int Hk, int N, int vfirst) {
  constexpr int KP = DK + 4, MT = DK / 16, NT = (MT + 3) / 4, NW = MT < 4 ? MT : 4;
  constexpr int NCT = NS / 16;           // 16-column tiles of the slice
  constexpr int NE = kC * NS / kThr;     // (token, column) elements per thread
  static_assert(NS % 16 == 0 && DV % NS == 0 && (kC * NS) % kThr == 0, "slice width");
  __shared__ __align__(16) float kh[kC][KP], qh[kC][KP];
  __shared__ __align__(16) float gs[CH ? kC + 1 : 1][CH ? KP : 4];
  __shared__ __align__(16) float TmT[kC][kCP], PmT[kC][kCP];
  __shared__ float part[NW][kC][NS + 1];
  __shared__ float dO[kC][NS + 1], dD[kC][NS + 1], BB[2 * kC][NS + 1];
  __shared__ TokVec tv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, li = lane & 15, lg = lane >> 4;
  constexpr int nsl = DV / NS;
  const int sl = blockIdx.x % nsl, bh = blockIdx.x / nsl, b = bh / H, h = bh % H, hk = h / (H / Hk);
  const int n0 = sl * NS;
  const long sb = static_cast<long>(bh) * DK * DV;
  auto sidx = [&](int c, int n) { return sb + (vfirst ? static_cast<long>(n) * DK + c : static_cast<long>(c) * DV + n); };
  f32x4 acc[NT][NCT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int mt = wave + 4 * j;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc[j][ct][e] = (mt < MT && dfinal) ? dfinal[sidx(16 * mt + 4 * lg + e, n0 + 16 * ct + li)] : 0.f;
    }
  }
  RowPf<DK, In, kThr> kpf, qpf;
  MatPf<kThr, true> mpf;
  TokPf tpf;
  GamPf<CH ? DK : 4, kThr> gpf;
  if (CH)
    for (int c = tid; c < DK; c += kThr) gs[0][c] = 0.f;
  float dov[NE];
  auto prefetch = [&](int c) __attribute__((always_inline)) {
    const int L = min(kC, T - c * kC);
    const long tok0 = static_cast<long>(b) * T + c * kC;
    kpf.load(k, w.sk, tok0, H, h, Hk, hk, L, tid);
    qpf.load(q, w.sq, tok0, H, h, Hk, hk, L, tid);
    mpf.load(w, (static_cast<size_t>(bh) * N + c) * kC * kC, tid);
    tpf.load(w, tok0, H, h, L, tid);
    if constexpr (CH) gpf.load(w.gmc, tok0, H, h, L, tid);
#pragma unroll
    for (int u = 0; u < NE; ++u) {
      const int idx = tid + u * kThr, r = min(idx / NS, L - 1), n = idx % NS;
      dov[u] = dout[((tok0 + r) * H + h) * DV + n0 + n];
    }
  };
  prefetch(N - 1);
  for (int ci = N - 1; ci >= 0; --ci) {
    const int t0 = ci * kC, L = min(kC, T - t0);
    const long tok0 = static_cast<long>(b) * T + t0;
    lds_sync();
    kpf.store(kh, L, tid);
    qpf.store(qh, L, tid);
    mpf.store(nullptr, TmT, PmT, tid);
    tpf.store<CH>(tv, L, tid);
    if constexpr (CH) gpf.store(gs, tid);
#pragma unroll
    for (int u = 0; u < NE; ++u) {
      const int idx = tid + u * kThr;
      dO[idx / NS][idx % NS] = idx / NS < L ? dov[u] : 0.f;
    }
    float* d1 = w.dS1 + (static_cast<size_t>(bh) * N + ci) * DK * DV;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int mt = wave + 4 * j;
      if (mt < MT) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
          for (int e = 0; e < 4; ++e) d1[(16 * mt + 4 * lg + e) * DV + n0 + 16 * ct + li] = acc[j][ct][e];
        }
      }
    }
    lds_sync();
    if (ci > 0) prefetch(ci - 1);
    // K dS over this wave's key rows
    if (wave < NW) {
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        f32x4 p[NCT];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) p[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          const int mt = wave + 4 * j;
          if (mt < MT) {
            f32x4 a = *reinterpret_cast<const f32x4*>(&kh[16 * rt + li][16 * mt + 4 * lg]);
            if constexpr (CH) {
              // k exp(gC - gam) per channel
              const f32x4 gm = *reinterpret_cast<const f32x4*>(&gs[16 * rt + li + 1][16 * mt + 4 * lg]);
              const f32x4 gC = *reinterpret_cast<const f32x4*>(&gs[L][16 * mt + 4 * lg]);
#pragma unroll
              for (int e = 0; e < 4; ++e) a[e] *= __expf(gC[e] - gm[e]);
            }
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
              for (int e = 0; e < 4; ++e) p[ct] = mma4(a[e], acc[j][ct][e], p[ct]);
            }
          }
        }
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
          for (int e = 0; e < 4; ++e) part[wave][16 * rt + 4 * lg + e][16 * ct + li] = p[ct][e];
        }
      }
    }
    // P^T dO into dD's place, a (row tile, column tile) per wave; (P^T)_rt =
    // P_tr vanishes for t < r: row tile 1 takes tokens 16.. only
    if (wave < 2 * NCT) {
      const int rt = wave & 1, ct = wave >> 1;
      f32x4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < kC / 16; ++kb) {
        if (kb >= rt) {
          const f32x4 a = *reinterpret_cast<const f32x4*>(&PmT[16 * rt + li][16 * kb + 4 * lg]);
#pragma unroll
          for (int e = 0; e < 4; ++e) p = mma4(a[e], dO[16 * kb + 4 * lg + e][16 * ct + li], p);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) dD[16 * rt + 4 * lg + e][16 * ct + li] = p[e];
    }
    lds_sync();
    if constexpr (CH) {
      // the rows of the dS update: q exp(gam) and k exp(gx), in place.  Row r
      // of gs is gx of token r and gam of token r - 1, so a thread that takes
      // one channel over consecutive tokens forms each exponential once.
      constexpr int TPC = kThr / DK;           // threads per channel
      static_assert(kThr % DK == 0 && kC % TPC == 0, "token runs per thread");
      constexpr int RUN = kC / TPC;
      const int c = tid % DK, r0 = (tid / DK) * RUN;
      float e0 = __expf(gs[r0][c]);
#pragma unroll
      for (int t = 0; t < RUN; ++t) {
        const int r = r0 + t;
        const float e1 = __expf(gs[r + 1][c]);
        kh[r][c] *= e0;
        qh[r][c] *= e1;
        e0 = e1;
      }
    }
    // dD = P^T dO + F . K dS; exp(gam) . dO, the update's first B operand
#pragma unroll
    for (int u = 0; u < NE; ++u) {
      const int idx = tid + u * kThr, r = idx / NS, n = idx % NS;
      float kd = 0.f;
#pragma unroll
      for (int qq = 0; qq < NW; ++qq) kd += part[qq][r][n];
      dD[r][n] += tv.F[r] * kd;
      BB[r][n] = tv.egm[r] * dO[r][n];
    }
    lds_sync();
    // dX = beta . T^T dD on MFMA (a row tile and column tile per wave; T^T is
    // upper triangular), the gradient of v, and the update's second B operand
    if (wave < 2 * NCT) {
      const int rt = wave & 1, ct = wave >> 1;
      f32x4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < kC / 16; ++kb) {
        if (kb >= rt) {
          const f32x4 a = *reinterpret_cast<const f32x4*>(&TmT[16 * rt + li][16 * kb + 4 * lg]);
#pragma unroll
          for (int e = 0; e < 4; ++e) p = mma4(a[e], dD[16 * kb + 4 * lg + e][16 * ct + li], p);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * rt + 4 * lg + e, n = 16 * ct + li;
        const float x = tv.bt[r] * p[e];
        if (r < L) dv[((tok0 + r) * H + h) * DV + n0 + n] = x;
        BB[kC + r][n] = -tv.egx[r] * x;
      }
    }
    lds_sync();
    // dS <- exp(gC) dS + Q^T (exp(gam) . dO) - K^T (exp(gx) . dX)
    const float egC = tv.egC;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int mt = wave + 4 * j;
      if (mt < MT) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          if constexpr (CH) {
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[j][ct][e] *= __expf(gs[L][16 * mt + 4 * lg + e]);
          } else {
            acc[j][ct] *= egC;
          }
        }
#pragma unroll
        for (int ks = 0; ks < kC / 4; ++ks) {
          const float qa = qh[4 * ks + lg][16 * mt + li];
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) acc[j][ct] = mma4(qa, BB[4 * ks + lg][16 * ct + li], acc[j][ct]);
        }
#pragma unroll
        for (int ks = 0; ks < kC / 4; ++ks) {
          const float ka = kh[4 * ks + lg][16 * mt + li];
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) acc[j][ct] = mma4(ka, BB[kC + 4 * ks + lg][16 * ct + li], acc[j][ct]);
        }
      }
    }
  }
  if (dinit) {
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int mt = wave + 4 * j;
      if (mt < MT) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
          for (int e = 0; e < 4; ++e) dinit[sidx(16 * mt + 4 * lg + e, n0 + 16 * ct + li)] = acc[j][ct][e];
        }
      }
    }
  }
}

// LDS of the per-chunk gradient kernel: the value-slice arrays and the last
// phase's matrices share their space.
template <int DK>
struct LocalLds {
  float kh[kC][DK + 4], qh[kC][DK + 4];
  float TmT[kC][kCP], PmT[kC][kCP];
  union {
    struct {
      float S0s[DK][kNS + 1], S1s[DK][kNS + 1];
      float KS[kC][kNS + 1], QS[kC][kNS + 1], KD[kC][kNS + 1];
      float dO[kC][kNS + 1], Yb[kC][kNS + 1], D[kC][kNS + 1], FD[kC][kNS + 1], dD[kC][kNS + 1];
      float dYs[kC][kNS + 1];
    } s;
    struct {
      float dTm[kC][kCP], M[kC][kCP];
      float dPm[kC][kC + 1], EE[kC][kC + 1], PP[kC][kC + 1], Gp[2][kC][kC + 1], dGs[kC][kC + 1];
      float nd[2][DK / 16][kC];   // the norm's row dots, per 16 key channels
      float fq[kC], fk[kC];       // the rows' norm factors
    } f;
  } u;
  float tb[kC], tm[kC], tx[kC], tc[kC], sgm[kC], sgx[kC], red[8];
  TokVec tv;
};

// (3) per (b, h, chunk): the remaining gradients over the value columns, 16
// at a time: dq and dk (through the norm and the scale; with grouped value
// heads those of the normalised rows, added up over the group), dbeta and the
// decay's gradient (written).  Eight waves, two workgroups per CU.  Per
// slice: K S0, Q S0, K dS1 and P^T dO on MFMA (one product's row tile per
// wave); X, Y and dD on VALU, one (row, column) element per thread; D = T Y
// and dY = T^T dD on MFMA (waves 0-3); the per-token sums on VALU; then on
// MFMA the running sums dT += dD Y^T, dP += dO D^T (a tile per wave) and
// dq += dO S0^T, dk += (F . D) dS1^T - (exp(gx) beta . dY) S0^T (tiles per
// wave, held across the slices).  Then M = dT T^T and -T^T M on MFMA; dA,
// dG and Z on VALU; and the last products dq += Z K, dk += (dG + dG^T) K +
// Z^T Q on MFMA.
template <int DK, int DV, typename In>
__global__ __launch_bounds__(kThr3, 4) void cbwd_local(const In* __restrict__ q, const In* __restrict__ k,
                                                       const In* __restrict__ v, const float* __restrict__ dout,
                                                       float* __restrict__ dq, float* __restrict__ dk,
                                                       float* __restrict__ dbeta, float* __restrict__ ddecay,
                                                       CWs w, int T, int H, int Hk, int N, float scale,
                                                       int l2norm) {
  constexpr int NT16 = DK / 16;
  constexpr int NQK = 4 * NT16, TPW = (NQK + 7) / 8;              // dq/dk tiles, per wave
  constexpr int SPT = DK * kNS / kThr3;                          // state floats per thread per slice
  constexpr int SL = kNS / SPT;                                   // threads per state row
  constexpr int nsl = DV / kNS;
  __shared__ __align__(16) LocalLds<DK> sm;
  auto& S = sm.u.s;
  auto& Fm = sm.u.f;
  TokVec& tv = sm.tv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, li = lane & 15, lg = lane >> 4;
  const int er = tid / kNS, en = tid % kNS;   // this thread's element of a 32 x 16 slice tile
  const int ci = blockIdx.x % N, bh = blockIdx.x / N, b = bh / H, h = bh % H, hk = h / (H / Hk);
  const int t0 = ci * kC, L = min(kC, T - t0);
  const long tok0 = static_cast<long>(b) * T + t0;
  const size_t cb = (static_cast<size_t>(bh) * N + ci) * kC * kC;
  const float* s0g = w.S0 + (static_cast<size_t>(bh) * N + ci) * DK * DV;
  const float* s1g = w.dS1 + (static_cast<size_t>(bh) * N + ci) * DK * DV;
  const bool rin = er < L;
  const int sc = tid / SL, sn = (tid % SL) * SPT;   // this thread's state elements: row sc, columns sn..
  const long vrowc = ((tok0 + min(er, L - 1)) * H + h) * DV;   // clamped: loads stay in range
  float ps0[SPT], ps1[SPT], pdo;
  typename Raw<In>::one pv;
  auto prefetch = [&](int s) __attribute__((always_inline)) {
    const int nb = s * kNS;
#pragma unroll
    for (int e = 0; e < SPT; ++e) {
      ps0[e] = s0g[sc * DV + nb + sn + e];
      ps1[e] = s1g[sc * DV + nb + sn + e];
    }
    pdo = dout[vrowc + nb + en];
    pv = Raw<In>::ld1(v + vrowc + nb + en);
  };
  prefetch(0);
  {
    RowPf<DK, In, kThr3> kpf, qpf;
    MatPf<kThr3, true> mpf;
    TokPf tpf;
    kpf.load(k, w.sk, tok0, H, h, Hk, hk, L, tid);
    qpf.load(q, w.sq, tok0, H, h, Hk, hk, L, tid);
    mpf.load(w, cb, tid);
    tpf.load(w, tok0, H, h, L, tid);
    kpf.store(sm.kh, L, tid);
    qpf.store(sm.qh, L, tid);
    mpf.store(nullptr, sm.TmT, sm.PmT, tid);
    tpf.store(tv, L, tid);
    if (tid < kC) {
      sm.sgm[tid] = tid < L ? tpf.gm : 0.f;
      sm.sgx[tid] = tid < L ? tpf.gx : 0.f;
    }
  }
  float sb = 0.f, so = 0.f, sx = 0.f, sf = 0.f, sdc = 0.f;   // per-token sums (this thread's columns)
  f32x4 atp = {0.f, 0.f, 0.f, 0.f};                          // dT (waves 0-3) or dP (4-7) tile
  f32x4 aqk[TPW];
#pragma unroll
  for (int j = 0; j < TPW; ++j) aqk[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int tpm = wave >> 2, tpr = (wave >> 1) & 1, tpc = wave & 1;
  const int prod = wave >> 1, prt = wave & 1;                // K-S products: which, row tile
  for (int s = 0; s < nsl; ++s) {
    lds_sync();
#pragma unroll
    for (int e = 0; e < SPT; ++e) {
      S.S0s[sc][sn + e] = ps0[e];
      S.S1s[sc][sn + e] = ps1[e];
      sdc += ps0[e] * ps1[e];
    }
    const float vcur = rin ? Raw<In>::cvt1(pv) : 0.f, docur = rin ? pdo : 0.f;
    S.dO[er][en] = docur;
    lds_sync();
    if (s + 1 < nsl) prefetch(s + 1);
    // K S0 (waves 0, 1), Q S0 (2, 3), K dS1 (4, 5): one row tile over all
    // keys; P^T dO (6, 7) into dD's place
    if (prod < 3) {
      const float(*A)[DK + 4] = prod == 1 ? sm.qh : sm.kh;
      const float(*Bm)[kNS + 1] = prod == 2 ? S.S1s : S.S0s;
      f32x4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
      for (int kb = 0; kb < DK / 16; ++kb) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(&A[16 * prt + li][16 * kb + 4 * lg]);
#pragma unroll
        for (int e = 0; e < 4; ++e) p = mma4(a[e], Bm[16 * kb + 4 * lg + e][li], p);
      }
      float(*O)[kNS + 1] = prod == 0 ? S.KS : (prod == 1 ? S.QS : S.KD);
#pragma unroll
      for (int e = 0; e < 4; ++e) O[16 * prt + 4 * lg + e][li] = p[e];
    } else {
      // (P^T)_rt = P_tr vanishes for t < r: row tile 1 takes tokens 16.. only
      f32x4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < kC / 16; ++kb) {
        if (kb >= prt) {
          const f32x4 a = *reinterpret_cast<const f32x4*>(&sm.PmT[16 * prt + li][16 * kb + 4 * lg]);
#pragma unroll
          for (int e = 0; e < 4; ++e) p = mma4(a[e], S.dO[16 * kb + 4 * lg + e][li], p);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) S.dD[16 * prt + 4 * lg + e][li] = p[e];
    }
    lds_sync();
    // X = V - exp(gx) . K S0, Y = beta . X;  dD = P^T dO + F . K dS1
    const float ksv = S.KS[er][en], kdv = S.KD[er][en];
    const float xo = tv.egx[er] * ksv, x = vcur - xo;
    S.Yb[er][en] = tv.bt[er] * x;
    S.dD[er][en] += tv.F[er] * kdv;
    so += docur * S.QS[er][en];
    lds_sync();
    // D = T Y (waves 0, 1) and dY = T^T dD (2, 3), a row tile each; raw dY
    // goes over K S0 (read above).  T is lower triangular: T Y's row tile 0
    // takes tokens 0..15 only, T^T dD's row tile 1 tokens 16.. only.
    if (wave < 2) {
      f32x4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < kC / 16; ++kb) {
        if (kb <= prt) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            p = mma4(sm.TmT[16 * kb + 4 * lg + e][16 * prt + li], S.Yb[16 * kb + 4 * lg + e][li], p);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * prt + 4 * lg + e;
        S.D[r][li] = p[e];
        S.FD[r][li] = tv.F[r] * p[e];
      }
    } else if (wave < 4) {
      f32x4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < kC / 16; ++kb) {
        if (kb >= prt) {
          const f32x4 a = *reinterpret_cast<const f32x4*>(&sm.TmT[16 * prt + li][16 * kb + 4 * lg]);
#pragma unroll
          for (int e = 0; e < 4; ++e) p = mma4(a[e], S.dD[16 * kb + 4 * lg + e][li], p);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * prt + 4 * lg + e;
        S.KS[r][li] = p[e];
        S.dYs[r][li] = -tv.egx[r] * tv.bt[r] * p[e];
      }
    }
    lds_sync();
    // the per-token sums
    const float d = S.D[er][en], y = S.KS[er][en];
    sb += y * x;
    sx += y * xo;
    sf += kdv * d;
    // dT += dD Y^T, dP += dO D^T (this wave's tile)
#pragma unroll
    for (int ks = 0; ks < kNS / 4; ++ks) {
      const float a = tpm ? S.dO[16 * tpr + li][4 * ks + lg] : S.dD[16 * tpr + li][4 * ks + lg];
      const float bb = tpm ? S.D[16 * tpc + li][4 * ks + lg] : S.Yb[16 * tpc + li][4 * ks + lg];
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
            aqk[j] = mma4(S.dO[r][n], S.S0s[c][n], aqk[j]);
          } else {
            aqk[j] = mma4(S.FD[r][n], S.S1s[c][n], aqk[j]);
            aqk[j] = mma4(S.dYs[r][n], S.S0s[c][n], aqk[j]);
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
  lds_sync();   // the slice arrays are dead from here: the last phase's matrices take their space
  if (en == 0) {
    sm.tb[er] = sb;
    sm.tm[er] = tv.egm[er] * so - tv.F[er] * sf;
    sm.tx[er] = -tv.bt[er] * sx;
    sm.tc[er] = tv.F[er] * sf;
  }
  if (lane == 0) sm.red[wave] = sdc;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int r = 16 * tpr + 4 * lg + e, c = 16 * tpc + li;
    if (tpm) Fm.dPm[r][c] = atp[e];
    else Fm.dTm[r][c] = c <= r ? atp[e] : 0.f;
  }
  lds_sync();
  // M = dT T^T (a tile per wave, waves 0-3) and K K^T on MFMA
  if (wave < 4) {
    const f32x4 p = tile_dt_tt(Fm.dTm, sm.TmT, wave >> 1, wave & 1, li, lg);
#pragma unroll
    for (int e = 0; e < 4; ++e) Fm.M[16 * (wave >> 1) + 4 * lg + e][16 * (wave & 1) + li] = p[e];
  }
  {
    const int gt = wave & 3, gr = gt >> 1, gc = gt & 1, gh = wave >> 2;
    f32x4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int kb = gh * (DK / 32); kb < (gh + 1) * (DK / 32); ++kb) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(&sm.kh[16 * gr + li][16 * kb + 4 * lg]);
      const f32x4 bq = *reinterpret_cast<const f32x4*>(&sm.kh[16 * gc + li][16 * kb + 4 * lg]);
#pragma unroll
      for (int e = 0; e < 4; ++e) p = mma4(a[e], bq[e], p);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) Fm.Gp[gh][16 * gr + 4 * lg + e][16 * gc + li] = p[e];
  }
  lds_sync();
  // -T^T M on MFMA, over dT (dead)
  if (wave < 4) {
    const f32x4 p = tile_tt_m(sm.TmT, Fm.M, wave >> 1, wave & 1, li, lg);
#pragma unroll
    for (int e = 0; e < 4; ++e) Fm.dTm[16 * (wave >> 1) + 4 * lg + e][16 * (wave & 1) + li] = -p[e];
  }
  lds_sync();
  // dA = -T^T M on s < r; E = dA . (K K^T) . W; dG = diag(beta) dA . W;
  // Z = dP . Vw (into dPm) and dP . P
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int idx = tid + u * kThr3, r = idx / kC, c = idx % kC;
    float e = 0.f, dg = 0.f;
    if (c < r) {
      const float da = Fm.dTm[r][c];
      const float wr = __expf(sm.sgx[r] - sm.sgm[c]);
      e = da * (Fm.Gp[0][r][c] + Fm.Gp[1][r][c]) * wr;
      dg = da * tv.bt[r] * wr;
    }
    Fm.EE[r][c] = e;
    Fm.Gp[0][r][c] = dg;   // this thread's own element of Gp, read above: dG in its place
    const float dp = c <= r ? Fm.dPm[r][c] : 0.f;
    Fm.PP[r][c] = dp * sm.PmT[c][r];
    Fm.dPm[r][c] = c <= r ? dp * __expf(sm.sgm[r] - sm.sgm[c]) : 0.f;
  }
  lds_sync();
  if (tid < kC) {
    const int r = tid;
    float re = 0.f, rp = 0.f, ce = 0.f, cp = 0.f;
#pragma unroll 8
    for (int t = 0; t < kC; ++t) {
      re += Fm.EE[r][t];
      rp += Fm.PP[r][t];
      ce += tv.bt[t] * Fm.EE[t][r];
      cp += Fm.PP[t][r];
    }
    sm.tb[r] += re;
    sm.tx[r] += tv.bt[r] * re;
    sm.tm[r] += rp - ce - cp;
    const long ti = (tok0 + min(r, L - 1)) * H + h;
    Fm.fq[r] = w.sq[ti];
    Fm.fk[r] = w.sk[ti];
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int idx = tid + u * kThr3, r = idx / kC, c = idx % kC;
    Fm.dGs[r][c] = Fm.Gp[0][r][c] + Fm.Gp[0][c][r];
  }
  lds_sync();
  // dq = exp(gam) . (dO S0^T) + Z K;  dk += (dG + dG^T) K + Z^T Q.  Without
  // grouped heads a row's gradient is whole here: the norm's backward
  // follows (the row dot with the unit row through LDS); with them the rows
  // are added up over the group and a last kernel takes the norm.
  const bool grouped = H != Hk;
#pragma unroll
  for (int j = 0; j < TPW; ++j) {
    const int t = wave + 8 * j;
    if (t < NQK) {
      const int mat = t / (2 * NT16), rem = t % (2 * NT16), mt = rem / NT16, nt = rem % NT16;
      f32x4& a = aqk[j];
      if (mat == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) a[e] *= tv.egm[16 * mt + 4 * lg + e];
#pragma unroll
        for (int ks = 0; ks < kC / 4; ++ks)
          a = mma4(Fm.dPm[16 * mt + li][4 * ks + lg], sm.kh[4 * ks + lg][16 * nt + li], a);
      } else {
#pragma unroll
        for (int ks = 0; ks < kC / 4; ++ks) {
          a = mma4(Fm.dGs[16 * mt + li][4 * ks + lg], sm.kh[4 * ks + lg][16 * nt + li], a);
          a = mma4(Fm.dPm[4 * ks + lg][16 * mt + li], sm.qh[4 * ks + lg][16 * nt + li], a);
        }
      }
      float* out = mat == 0 ? dq : dk;
      if (grouped) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * mt + 4 * lg + e;
          if (r < L) atomicAdd(out + ((tok0 + r) * Hk + hk) * DK + 16 * nt + li, a[e]);
        }
      } else {
        // unit row: q's normalised row is qh / scale, k's is kh
        const float xs = l2norm ? (mat == 0 ? 1.f / scale : 1.f) : 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * mt + 4 * lg + e;
          const float xr = (mat == 0 ? sm.qh[r][16 * nt + li] : sm.kh[r][16 * nt + li]) * xs;
          const float pd = dpp_group_sum<16>(xr * a[e]);
          if (li == 0) Fm.nd[mat][nt][r] = pd;
        }
      }
    }
  }
  if (!grouped) {
    lds_sync();
    // g_raw = f (g - x (x . g)), f the row's norm factor (scale / |x| for q)
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      const int t = wave + 8 * j;
      if (t < NQK) {
        const int mat = t / (2 * NT16), rem = t % (2 * NT16), mt = rem / NT16, nt = rem % NT16;
        float* out = mat == 0 ? dq : dk;
        const float xs = l2norm ? (mat == 0 ? 1.f / scale : 1.f) : 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * mt + 4 * lg + e;
          if (r < L) {
            float dot = 0.f;
#pragma unroll
            for (int u = 0; u < NT16; ++u) dot += Fm.nd[mat][u][r];
            const float xr = (mat == 0 ? sm.qh[r][16 * nt + li] : sm.kh[r][16 * nt + li]) * xs;
            const float f = mat == 0 ? Fm.fq[r] : Fm.fk[r];
            out[((tok0 + r) * Hk + hk) * DK + 16 * nt + li] = f * (aqk[j][e] - xr * dot);
          }
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
      for (int wv = 0; wv < 8; ++wv) dgc += sm.red[wv];
      dgc *= tv.egC;
#pragma unroll 8
      for (int r = 0; r < kC; ++r) {
        dgc += sm.tc[r];
        if (r >= t) sg += sm.tm[r];
        if (r > t) sg += sm.tx[r];
      }
      const long ti = (tok0 + t) * H + h;
      dbeta[ti] = sm.tb[t];
      if (ddecay) ddecay[ti] = sg + dgc;
    }
  }
}

// (0) per-channel decay: per (b, h, chunk) the norm factors of the rows,
// beta, gam per key channel (to the workspace), and T and P of the chunk,
// each Gram entry summed over the channels with its own decay factor
// exp(gx_rc - gam_sc) (A) or exp(gam_rc - gam_sc) (P), every exponent <= 0.
template <int DK, typename In>
__global__ __launch_bounds__(kThr) void cbwd_prep_ch(const In* __restrict__ q, const In* __restrict__ k,
                                                     const In* __restrict__ beta, const In* __restrict__ decay,
                                                     CWs w, int T, int H, int Hk, int N, float scale, int l2norm,
                                                     Transforms tf) {
  constexpr int KP = DK + 4;
  __shared__ __align__(16) float kh[kC][KP], qh[kC][KP];
  __shared__ __align__(16) float gs[kC + 1][KP];   // row r + 1: gam of token r; row 0: zeros
  __shared__ __align__(16) float sA[kC][kCP];
  __shared__ float sbt[kC];
  const int tid = threadIdx.x;
  const int ci = blockIdx.x % N, bh = blockIdx.x / N, b = bh / H, h = bh % H, hk = h / (H / Hk);
  const int t0 = ci * kC, L = min(kC, T - t0);
  const long tok0 = static_cast<long>(b) * T + t0;
  const float negA = tf.A_log ? -__expf(tf.A_log[h]) : 0.f;
  {
    constexpr int V = act<In>::kVec, LPR = DK / V;
    static_assert(kC * LPR % 64 == 0, "whole waves per pass");
    for (int idx = tid; idx < kC * LPR; idx += kThr) {
      const int r = idx / LPR, seg = idx % LPR;
      const bool in = r < L;
      float qv[V], kv[V], gv[V], sq = 0.f, sk = 0.f;
      if (in) {
        const long base = ((tok0 + r) * Hk + hk) * DK + seg * V;
        act<In>::load_vec(q + base, qv);
        act<In>::load_vec(k + base, kv);
        act<In>::load_vec(decay + ((tok0 + r) * H + h) * DK + seg * V, gv);
        if (tf.A_log) {
#pragma unroll
          for (int e = 0; e < V; ++e)
            gv[e] = gate_decay(gv[e], negA, tf.dt_bias ? tf.dt_bias[h * DK + seg * V + e] : 0.f, tf.lower);
        }
      } else {
#pragma unroll
        for (int e = 0; e < V; ++e) qv[e] = kv[e] = gv[e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < V; ++e) {
        sq += qv[e] * qv[e];
        sk += kv[e] * kv[e];
      }
      sq = dpp_group_sum<LPR>(sq);
      sk = dpp_group_sum<LPR>(sk);
      const float fq = (l2norm ? inv_norm(sq) : 1.f) * scale, fk = l2norm ? inv_norm(sk) : 1.f;
#pragma unroll
      for (int e = 0; e < V; ++e) {
        qh[r][seg * V + e] = qv[e] * fq;
        kh[r][seg * V + e] = kv[e] * fk;
        gs[r + 1][seg * V + e] = gv[e];
      }
      if (seg == 0 && in) {
        w.sq[(tok0 + r) * H + h] = fq;
        w.sk[(tok0 + r) * H + h] = fk;
      }
    }
  }
  if (tid < kC) {
    const bool in = tid < L;
    const long ti = (tok0 + tid) * H + h;
    const float bt = in ? beta_transform(act<In>::load1(beta + ti), tf.beta_mode) : 0.f;
    sbt[tid] = bt;
    if (in) w.bt[ti] = bt;
  }
  lds_sync();
  // gam per channel: a running sum down the chunk's tokens (past the end the
  // decay is zero, so the last token's value repeats)
  for (int c = tid; c < DK; c += kThr) {
    float acc = 0.f;
    gs[0][c] = 0.f;
    for (int r = 0; r < kC; ++r) {
      acc += gs[r + 1][c];
      gs[r + 1][c] = acc;
      if (r < L) w.gmc[((tok0 + r) * H + h) * DK + c] = acc;
    }
  }
  lds_sync();
  const size_t cb = (static_cast<size_t>(bh) * N + ci) * kC * kC;
  // Entries s <= r.  Token s of the first 16 against token r of the last 16:
  // exp(gx_r - gam_s) = exp(gx_r - gam_15) exp(gam_15 - gam_s) and
  // exp(gam_r - gam_s) = exp(gam_r - gam_15) exp(gam_15 - gam_s), each factor
  // <= 1, so that block is a product of decayed rows on MFMA (wave 0, A and
  // P together).  Within each diagonal block the same split at the last
  // token of its first half gives the later half's rows against the earlier
  // half's tokens (wave 1, both blocks in one product).  The four 8-token
  // halves' 36 pairs each: one pair per thread of waves 2 and 3, the channel
  // sum with its own factors.
  if (tid < 64) {
    const int li = tid & 15, lg = tid >> 4;
    f32x4 aa = {0.f, 0.f, 0.f, 0.f}, pa = aa;
#pragma unroll 4
    for (int ks = 0; ks < DK / 4; ++ks) {
      const int c = 4 * ks + lg;
      const float g15 = gs[16][c];
      const float bk = kh[li][c] * __expf(g15 - gs[li + 1][c]);                 // k_s exp(gam_15 - gam_s)
      const float ak = kh[16 + li][c] * __expf(gs[16 + li][c] - g15);           // k_r exp(gx_r - gam_15)
      const float aq = qh[16 + li][c] * __expf(gs[17 + li][c] - g15);           // q_r exp(gam_r - gam_15)
      aa = mma4(ak, bk, aa);
      pa = mma4(aq, bk, pa);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 + 4 * lg + e, s2 = li;
      sA[r][s2] = sbt[r] * aa[e];
      w.Pm[cb + r * kC + s2] = pa[e];
    }
  } else if (tid < 128) {
    // tile row / column i: block i >> 3, token 16 (i >> 3) + 8 + (i & 7) (rows)
    // or 16 (i >> 3) + (i & 7) (columns); entries across the two blocks are
    // not kept
    const int li = tid & 15, lg = (tid >> 4) & 3;
    const int rr = 16 * (li >> 3) + 8 + (li & 7), sc = 16 * (li >> 3) + (li & 7);
    f32x4 aa = {0.f, 0.f, 0.f, 0.f}, pa = aa;
#pragma unroll 4
    for (int ks = 0; ks < DK / 4; ++ks) {
      const int c = 4 * ks + lg;
      const float gr7 = gs[16 * (li >> 3) + 8][c];   // gam at the block's token 7 (row and column alike)
      const float bk = kh[sc][c] * __expf(gr7 - gs[sc + 1][c]);    // k_s exp(gam_7 - gam_s)
      const float ak = kh[rr][c] * __expf(gs[rr][c] - gr7);        // k_r exp(gx_r - gam_7)
      const float aq = qh[rr][c] * __expf(gs[rr + 1][c] - gr7);    // q_r exp(gam_r - gam_7)
      aa = mma4(ak, bk, aa);
      pa = mma4(aq, bk, pa);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int ti = 4 * lg + e;
      if ((ti >> 3) == (li >> 3)) {
        const int r = 16 * (ti >> 3) + 8 + (ti & 7);
        sA[r][sc] = sbt[r] * aa[e];
        w.Pm[cb + r * kC + sc] = pa[e];
      }
    }
  }
  // The 4 x 36 within-half pairs: one per thread of waves 2 and 3, the 16
  // left over on wave 1 once its product is done.
  static_assert(kThr == 256 && 4 * 36 - 128 <= 64, "pair jobs per thread");
  {
    const int idx = tid >= 128 ? tid - 128 : (tid >= 64 ? 128 + (tid - 64) : 4 * 36);
    if (idx < 4 * 36) {
      const int hf = idx / 36, id = idx % 36;   // half hf: tokens 8 hf .. 8 hf + 7
      int rl = static_cast<int>((sqrtf(8.f * id + 1.f) - 1.f) * 0.5f);
      if ((rl + 1) * (rl + 2) / 2 <= id) ++rl;
      if (rl * (rl + 1) / 2 > id) --rl;
      const int r = 8 * hf + rl, s = 8 * hf + id - rl * (rl + 1) / 2;
      float a0 = 0.f, a1 = 0.f, p0 = 0.f, p1 = 0.f;
#pragma unroll 4
      for (int c = 0; c < DK; c += 4) {
        const f32x4 kr = *reinterpret_cast<const f32x4*>(&kh[r][c]);
        const f32x4 ks = *reinterpret_cast<const f32x4*>(&kh[s][c]);
        const f32x4 qr = *reinterpret_cast<const f32x4*>(&qh[r][c]);
        const f32x4 gx = *reinterpret_cast<const f32x4*>(&gs[r][c]);
        const f32x4 gr = *reinterpret_cast<const f32x4*>(&gs[r + 1][c]);
        const f32x4 gsv = *reinterpret_cast<const f32x4*>(&gs[s + 1][c]);
#pragma unroll
        for (int e = 0; e < 4; e += 2) {
          p0 += qr[e] * ks[e] * __expf(gr[e] - gsv[e]);
          p1 += qr[e + 1] * ks[e + 1] * __expf(gr[e + 1] - gsv[e + 1]);
          // exp(gx_r - gam_s) <= 1 only for s < r: masked below
          a0 += kr[e] * ks[e] * __expf(fminf(gx[e] - gsv[e], 0.f));
          a1 += kr[e + 1] * ks[e + 1] * __expf(fminf(gx[e + 1] - gsv[e + 1], 0.f));
        }
      }
      sA[r][s] = s < r ? sbt[r] * (a0 + a1) : 0.f;
      w.Pm[cb + r * kC + s] = p0 + p1;
    }
  }
  // the upper triangles: zeros
  for (int idx = tid; idx < kC * kC; idx += kThr) {
    const int r = idx / kC, s = idx % kC;
    if (s > r) {
      sA[r][s] = 0.f;
      w.Pm[cb + idx] = 0.f;
    }
  }
  lds_sync();
  if (tid < kC) {
    // column j of T = (I + A)^-1
    const int j = tid;
    float x[kC];
    tri_inv_col(sA, j, x);
#pragma unroll
    for (int r = 0; r < kC; ++r) w.Tm[cb + r * kC + j] = x[r];
  }
}

// LDS of the per-chunk gradient kernel with a per-channel decay
template <int DK>
struct LocalChLds {
  float kh[kC][DK + 4], qh[kC][DK + 4];   // normalised rows
  float kx[kC][DK + 4], kf[kC][DK + 4];   // k exp(gx), k exp(gC - gam)
  float gs[kC + 1][DK + 4];               // row r + 1: gam of token r; row 0: zeros
  float TmT[kC][kCP], PmT[kC][kCP];
  union {
    struct {
      float S0s[DK][kNS + 1], S1s[DK][kNS + 1];
      float KX[kC][kNS + 1], KD[kC][kNS + 1];
      float dO[kC][kNS + 1], Yb[kC][kNS + 1], D[kC][kNS + 1], dX[kC][kNS + 1], dD[kC][kNS + 1];
    } s;
    struct {
      float dTm[kC][kCP], M[kC][kCP], dA[kC][kCP], dPm[kC][kCP];
      float Wg[kC][DK + 4];               // dgam_r + dgx_{r+1} per channel
      float dbp[DK / 16][kC];             // dbeta parts per 16 channels
      float dgcp[2][DK];                  // dgC parts per row tile
      float nd[2][DK / 16][kC];           // the norm's row dots, per 16 channels
      float fq[kC], fk[kC];               // the rows' norm factors
    } f;
  } u;
  float tb[kC], dgs[DK];
  TokVec tv;
};

// (3) per-channel decay, per (b, h, chunk): dq, dk (as in the per-head
// kernel), dbeta and the per-channel decay's gradient.  Per slice of 16 value
// columns: X = V - (k exp(gx)) S0 and K dS1 with F folded in, and P^T dO, on
// MFMA (one row tile per wave, waves 0-5); then D = T Y and dY = T^T dD on
// MFMA (waves 0-3); then the running sums
// dT, dP (a tile per wave) and, per (row, channel) position held by a wave,
// dO S0^T, dX S0^T and D dS1^T.  Then dA; then, at each position, the
// in-chunk pair terms (sums over the partner token u of dA or dP times k or
// q and the decay factor between u and the row, a product of per-token
// factors exp(g) <= 1 carried down or up the partners), and the gradients
// from them and the three sums.  The decay's gradient is a reverse running
// sum down the tokens per channel.
template <int DK, int DV, typename In>
__global__ __launch_bounds__(kThr3) void cbwd_local_ch(const In* __restrict__ q, const In* __restrict__ k,
                                                       const In* __restrict__ v, const float* __restrict__ dout,
                                                       float* __restrict__ dq, float* __restrict__ dk,
                                                       float* __restrict__ dbeta, float* __restrict__ ddecay,
                                                       CWs w, int T, int H, int Hk, int N, float scale,
                                                       int l2norm) {
  constexpr int NT16 = DK / 16, NPOS = 2 * NT16, PPW = (NPOS + 7) / 8;   // (row tile, channel tile) positions
  constexpr int SPT = DK * kNS / kThr3, SL = kNS / SPT, nsl = DV / kNS;
  __shared__ __align__(16) LocalChLds<DK> sm;
  auto& S = sm.u.s;
  auto& Fm = sm.u.f;
  TokVec& tv = sm.tv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, li = lane & 15, lg = lane >> 4;
  const int er = tid / kNS, en = tid % kNS;
  const int ci = blockIdx.x % N, bh = blockIdx.x / N, b = bh / H, h = bh % H, hk = h / (H / Hk);
  const int t0 = ci * kC, L = min(kC, T - t0);
  const long tok0 = static_cast<long>(b) * T + t0;
  const size_t cb = (static_cast<size_t>(bh) * N + ci) * kC * kC;
  const float* s0g = w.S0 + (static_cast<size_t>(bh) * N + ci) * DK * DV;
  const float* s1g = w.dS1 + (static_cast<size_t>(bh) * N + ci) * DK * DV;
  const bool rin = er < L;
  const long vrowc = ((tok0 + min(er, L - 1)) * H + h) * DV;
  const int sc = tid / SL, sn = (tid % SL) * SPT;
  float ps0[SPT], ps1[SPT], pdo;
  typename Raw<In>::one pv;
  auto prefetch = [&](int s) __attribute__((always_inline)) {
    const int nb = s * kNS;
#pragma unroll
    for (int e = 0; e < SPT; ++e) {
      ps0[e] = s0g[sc * DV + nb + sn + e];
      ps1[e] = s1g[sc * DV + nb + sn + e];
    }
    pdo = dout[vrowc + nb + en];
    pv = Raw<In>::ld1(v + vrowc + nb + en);
  };
  prefetch(0);
  {
    RowPf<DK, In, kThr3> kpf, qpf;
    MatPf<kThr3, true> mpf;
    TokPf tpf;
    GamPf<DK, kThr3> gpf;
    kpf.load(k, w.sk, tok0, H, h, Hk, hk, L, tid);
    qpf.load(q, w.sq, tok0, H, h, Hk, hk, L, tid);
    mpf.load(w, cb, tid);
    tpf.load(w, tok0, H, h, L, tid);
    gpf.load(w.gmc, tok0, H, h, L, tid);
    kpf.store(sm.kh, L, tid);
    qpf.store(sm.qh, L, tid);
    mpf.store(nullptr, sm.TmT, sm.PmT, tid);
    tpf.store<true>(tv, L, tid);
    gpf.store(sm.gs, tid);
    for (int c = tid; c < DK; c += kThr3) sm.gs[0][c] = 0.f;
  }
  lds_sync();
  for (int idx = tid; idx < kC * DK; idx += kThr3) {
    const int r = idx / DK, c = idx % DK;
    sm.kx[r][c] = sm.kh[r][c] * __expf(sm.gs[r][c]);
    sm.kf[r][c] = sm.kh[r][c] * __expf(sm.gs[L][c] - sm.gs[r + 1][c]);
  }
  float sb = 0.f, sdc = 0.f;
  f32x4 atp = {0.f, 0.f, 0.f, 0.f};
  f32x4 aq[PPW], ax[PPW], af[PPW];
#pragma unroll
  for (int j = 0; j < PPW; ++j) aq[j] = ax[j] = af[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int tpm = wave >> 2, tpr = (wave >> 1) & 1, tpc = wave & 1;
  const int prod = wave >> 1, prt = wave & 1;   // waves 0-3: K S0 (prod 0) or K dS1 (prod 1), row tile prt
  for (int s = 0; s < nsl; ++s) {
    lds_sync();
#pragma unroll
    for (int e = 0; e < SPT; ++e) {
      S.S0s[sc][sn + e] = ps0[e];
      S.S1s[sc][sn + e] = ps1[e];
      sdc += ps0[e] * ps1[e];
    }
    const float vcur = rin ? Raw<In>::cvt1(pv) : 0.f, docur = rin ? pdo : 0.f;
    S.dO[er][en] = docur;
    lds_sync();
    if (s + 1 < nsl) prefetch(s + 1);
    if (prod < 2) {
      const float(*A)[DK + 4] = prod == 0 ? sm.kx : sm.kf;
      const float(*Bm)[kNS + 1] = prod == 0 ? S.S0s : S.S1s;
      f32x4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
      for (int kb = 0; kb < DK / 16; ++kb) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(&A[16 * prt + li][16 * kb + 4 * lg]);
#pragma unroll
        for (int e = 0; e < 4; ++e) p = mma4(a[e], Bm[16 * kb + 4 * lg + e][li], p);
      }
      float(*O)[kNS + 1] = prod == 0 ? S.KX : S.KD;
#pragma unroll
      for (int e = 0; e < 4; ++e) O[16 * prt + 4 * lg + e][li] = p[e];
    } else if (prod == 2) {
      // P^T dO (waves 4, 5) into dD's place; (P^T)_rt = P_tr vanishes for
      // t < r: row tile 1 takes tokens 16.. only
      f32x4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < kC / 16; ++kb) {
        if (kb >= prt) {
          const f32x4 a = *reinterpret_cast<const f32x4*>(&sm.PmT[16 * prt + li][16 * kb + 4 * lg]);
#pragma unroll
          for (int e = 0; e < 4; ++e) p = mma4(a[e], S.dO[16 * kb + 4 * lg + e][li], p);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) S.dD[16 * prt + 4 * lg + e][li] = p[e];
    }
    lds_sync();
    const float x = vcur - S.KX[er][en];
    S.Yb[er][en] = tv.bt[er] * x;
    S.dD[er][en] += S.KD[er][en];
    lds_sync();
    // D = T Y (waves 0, 1) and dY = T^T dD (2, 3), a row tile each; raw dY
    // goes over K X (read above).  T is lower triangular: T Y's row tile 0
    // takes tokens 0..15 only, T^T dD's row tile 1 tokens 16.. only.
    if (wave < 2) {
      f32x4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < kC / 16; ++kb) {
        if (kb <= prt) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            p = mma4(sm.TmT[16 * kb + 4 * lg + e][16 * prt + li], S.Yb[16 * kb + 4 * lg + e][li], p);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) S.D[16 * prt + 4 * lg + e][li] = p[e];
    } else if (wave < 4) {
      f32x4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < kC / 16; ++kb) {
        if (kb >= prt) {
          const f32x4 a = *reinterpret_cast<const f32x4*>(&sm.TmT[16 * prt + li][16 * kb + 4 * lg]);
#pragma unroll
          for (int e = 0; e < 4; ++e) p = mma4(a[e], S.dD[16 * kb + 4 * lg + e][li], p);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * prt + 4 * lg + e;
        S.KX[r][li] = p[e];
        S.dX[r][li] = tv.bt[r] * p[e];
      }
    }
    lds_sync();
    sb += S.KX[er][en] * x;
#pragma unroll
    for (int ks = 0; ks < kNS / 4; ++ks) {
      const float a = tpm ? S.dO[16 * tpr + li][4 * ks + lg] : S.dD[16 * tpr + li][4 * ks + lg];
      const float bb = tpm ? S.D[16 * tpc + li][4 * ks + lg] : S.Yb[16 * tpc + li][4 * ks + lg];
      atp = mma4(a, bb, atp);
    }
#pragma unroll
    for (int j = 0; j < PPW; ++j) {
      const int pos = wave + 8 * j;
      if (pos < NPOS) {
        const int mt = pos / NT16, nt = pos % NT16;
#pragma unroll
        for (int ks = 0; ks < kNS / 4; ++ks) {
          const int r = 16 * mt + li, n = 4 * ks + lg, c = 16 * nt + li;
          const float b0 = S.S0s[c][n];
          aq[j] = mma4(S.dO[r][n], b0, aq[j]);
          ax[j] = mma4(S.dX[r][n], b0, ax[j]);
          af[j] = mma4(S.D[r][n], S.S1s[c][n], af[j]);
        }
      }
    }
  }
  sb = dpp_group_sum<16>(sb);
  // <dS1, S0> per key channel: the SL threads of a state row are consecutive lanes
  if constexpr (SL > 1) sdc = group_sum<SL>(sdc);
  lds_sync();
  // the per-token decay factors a_t = exp(g_t) per channel, in kx's place
  for (int idx = tid; idx < kC * DK; idx += kThr3) {
    const int t = idx / DK, c = idx % DK;
    sm.kx[t][c] = __expf(sm.gs[t + 1][c] - sm.gs[t][c]);
  }
  if (en == 0) sm.tb[er] = sb;
  if (tid % SL == 0) sm.dgs[sc] = __expf(sm.gs[L][sc]) * sdc;
  if (tid < kC) {
    const long ti = (tok0 + min(tid, L - 1)) * H + h;
    Fm.fq[tid] = w.sq[ti];
    Fm.fk[tid] = w.sk[ti];
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int r = 16 * tpr + 4 * lg + e, c = 16 * tpc + li;
    if (tpm) Fm.dPm[r][c] = c <= r ? atp[e] : 0.f;
    else Fm.dTm[r][c] = c <= r ? atp[e] : 0.f;
  }
  lds_sync();
  // M = dT T^T, then dA = -T^T M on s < r: a tile per wave, waves 0-3
  if (wave < 4) {
    const f32x4 p = tile_dt_tt(Fm.dTm, sm.TmT, wave >> 1, wave & 1, li, lg);
#pragma unroll
    for (int e = 0; e < 4; ++e) Fm.M[16 * (wave >> 1) + 4 * lg + e][16 * (wave & 1) + li] = p[e];
  }
  lds_sync();
  if (wave < 4) {
    const f32x4 p = tile_tt_m(sm.TmT, Fm.M, wave >> 1, wave & 1, li, lg);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 * (wave >> 1) + 4 * lg + e, c = 16 * (wave & 1) + li;
      Fm.dA[r][c] = c < r ? -p[e] : 0.f;
    }
  }
  lds_sync();
  // per position: the pair terms and the gradients; without grouped heads
  // the rows of dq and dk are whole here and the norm's backward follows
  const bool grouped = H != Hk;
  float dgx[PPW][4], oq[PPW][4], ok[PPW][4];
#pragma unroll
  for (int j = 0; j < PPW; ++j) {
    const int pos = wave + 8 * j;
    if (pos < NPOS) {
      const int mt = pos / NT16, nt = pos % NT16, c = 16 * nt + li;
      float G1[4] = {0.f, 0.f, 0.f, 0.f}, G2[4] = {0.f, 0.f, 0.f, 0.f};
      float H1[4] = {0.f, 0.f, 0.f, 0.f}, H2[4] = {0.f, 0.f, 0.f, 0.f};
      float gx[4], gm[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        gx[e] = sm.gs[16 * mt + 4 * lg + e][c];
        gm[e] = sm.gs[16 * mt + 4 * lg + e + 1][c];
      }
      // The decay factor between tokens u and r.  Partners in the row's own
      // 8-token half block: a product of the per-token factors a_t =
      // exp(g_t) <= 1 strictly between or up to them, carried down (u < r) and
      // up (u > r) the partner tokens (no exponential per pair, no factor
      // above one).  Partners in the other 16-token block, or in the other
      // half of the row's block: a product on MFMA, the decay split at the
      // last token of the earlier block or half into two factors <= 1
      // (exp(gx_r - gam_u) = exp(gx_r - gam_s) exp(gam_s - gam_u), and so on),
      // one on the partner's row, one applied to the result.
      if (mt == 1) {
        f32x4 g1 = {0.f, 0.f, 0.f, 0.f}, h1 = g1;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int u = 4 * ks + lg;
          const float b0 = sm.kh[u][c] * __expf(sm.gs[16][c] - sm.gs[u + 1][c]);   // k_u exp(gam_15 - gam_u)
          g1 = mma4(Fm.dA[16 + li][u], b0, g1);
          h1 = mma4(Fm.dPm[16 + li][u], b0, h1);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 + 4 * lg + e;
          G1[e] += g1[e] * __expf(sm.gs[r][c] - sm.gs[16][c]);
          H1[e] += h1[e] * __expf(sm.gs[r + 1][c] - sm.gs[16][c]);
        }
      } else {
        f32x4 g2 = {0.f, 0.f, 0.f, 0.f}, h2 = g2;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int u = 16 + 4 * ks + lg;
          const float bk = tv.bt[u] * sm.kh[u][c] * __expf(sm.gs[u][c] - sm.gs[16][c]);   // exp(gx_u - gam_15)
          const float bq = sm.qh[u][c] * __expf(sm.gs[u + 1][c] - sm.gs[16][c]);          // exp(gam_u - gam_15)
          g2 = mma4(Fm.dA[u][li], bk, g2);
          h2 = mma4(Fm.dPm[u][li], bq, h2);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float f = __expf(sm.gs[16][c] - sm.gs[4 * lg + e + 1][c]);   // exp(gam_15 - gam_r)
          G2[e] += g2[e] * f;
          H2[e] += h2[e] * f;
        }
      }
      // partners in the other half of the row's block: split at token s = 16 mt + 7
      {
        const float gh = sm.gs[16 * mt + 8][c];   // gam_s
        const bool hi = li >= 8;                  // the A operand's row in the later half
        f32x4 g1 = {0.f, 0.f, 0.f, 0.f}, h1 = g1, g2 = g1, h2 = g1;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int u1 = 16 * mt + 4 * ks + lg, u2 = u1 + 8, rr = 16 * mt + li;
          const float b1 = sm.kh[u1][c] * __expf(gh - sm.gs[u1 + 1][c]);                // k_u exp(gam_s - gam_u)
          const float bk = tv.bt[u2] * sm.kh[u2][c] * __expf(sm.gs[u2][c] - gh);        // exp(gx_u - gam_s)
          const float bq = sm.qh[u2][c] * __expf(sm.gs[u2 + 1][c] - gh);                // exp(gam_u - gam_s)
          g1 = mma4(hi ? Fm.dA[rr][u1] : 0.f, b1, g1);
          h1 = mma4(hi ? Fm.dPm[rr][u1] : 0.f, b1, h1);
          g2 = mma4(hi ? 0.f : Fm.dA[u2][rr], bk, g2);
          h2 = mma4(hi ? 0.f : Fm.dPm[u2][rr], bq, h2);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * mt + 4 * lg + e;
          if (lg >= 2) {
            G1[e] += g1[e] * __expf(sm.gs[r][c] - gh);       // exp(gx_r - gam_s)
            H1[e] += h1[e] * __expf(sm.gs[r + 1][c] - gh);   // exp(gam_r - gam_s)
          } else {
            const float f = __expf(gh - sm.gs[r + 1][c]);    // exp(gam_s - gam_r)
            G2[e] += g2[e] * f;
            H2[e] += h2[e] * f;
          }
        }
      }
      // partners in the row's own half block: running products (a lane's four
      // rows lie in one half, which starts at token hb)
      const int hb = 16 * mt + 8 * (lg >> 1);
      {
        float E1[4] = {1.f, 1.f, 1.f, 1.f}, E2[4] = {1.f, 1.f, 1.f, 1.f};
        // partners u <= r start at the half's last row
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
          const int uu = hb + 7 - kk;
          const float ku = sm.kh[uu][c], an = sm.kx[min(uu + 1, kC - 1)][c];   // a_{u+1}
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 16 * mt + 4 * lg + e;
            E1[e] = uu >= r - 1 ? 1.f : E1[e] * an;   // exp(gx_r - gam_u), u < r
            E2[e] = uu >= r ? 1.f : E2[e] * an;       // exp(gam_r - gam_u), u <= r
            G1[e] += Fm.dA[r][uu] * ku * E1[e];
            H1[e] += Fm.dPm[r][uu] * ku * E2[e];
          }
        }
      }
      {
        float E1[4] = {1.f, 1.f, 1.f, 1.f}, E2[4] = {1.f, 1.f, 1.f, 1.f};
        // partners u >= r start at the half's first row
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
          const int uu = hb + kk;
          const float ku = sm.kh[uu][c], qu = sm.qh[uu][c], bu = tv.bt[uu];
          const float ap = sm.kx[max(uu - 1, 0)][c], au = sm.kx[uu][c];   // a_{u-1}, a_u
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 16 * mt + 4 * lg + e;
            E1[e] = uu <= r + 1 ? 1.f : E1[e] * ap;   // exp(gx_u - gam_r), u > r
            E2[e] = uu <= r ? 1.f : E2[e] * au;       // exp(gam_u - gam_r), u >= r
            G2[e] += Fm.dA[uu][r] * bu * ku * E1[e];
            H2[e] += Fm.dPm[uu][r] * qu * E2[e];
          }
        }
      }
      float dbe[4], dgc = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * mt + 4 * lg + e;
        const float kr = sm.kh[r][c], qr = sm.qh[r][c], br = tv.bt[r];
        const float egm = __expf(gm[e]), egx = __expf(gx[e]), Fx = __expf(sm.gs[L][c] - gm[e]);
        const float dqv = egm * aq[j][e] + H1[e];
        const float dkv = -egx * ax[j][e] + Fx * af[j][e] + br * G1[e] + G2[e] + H2[e];
        const float kfa = kr * Fx * af[j][e];
        Fm.Wg[r][c] = qr * egm * aq[j][e] - kfa + qr * H1[e] - kr * (G2[e] + H2[e]);
        dgx[j][e] = -kr * egx * ax[j][e] + br * kr * G1[e];
        dbe[e] = kr * G1[e];
        dgc += kfa;
        oq[j][e] = dqv;
        ok[j][e] = dkv;
        if (grouped) {
          if (r < L) {
            const long o = ((tok0 + r) * Hk + hk) * DK + c;
            atomicAdd(dq + o, dqv);
            atomicAdd(dk + o, dkv);
          }
        } else {
          // row dots with the unit rows (qh / scale, kh)
          const float xq = l2norm ? qr / scale : 0.f, xk = l2norm ? kr : 0.f;
          const float pq = dpp_group_sum<16>(xq * dqv), pk = dpp_group_sum<16>(xk * dkv);
          if (li == 0) {
            Fm.nd[0][nt][r] = pq;
            Fm.nd[1][nt][r] = pk;
          }
        }
      }
      // dbeta: k G1 over the 16 channels of the tile; dgC: over the 16 rows
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dbe[e] = dpp_group_sum<16>(dbe[e]);
        if (li == 0) Fm.dbp[nt][16 * mt + 4 * lg + e] = dbe[e];
      }
      dgc = xor32_sum(xor16_sum(dgc));
      if (lg == 0) Fm.dgcp[mt][c] = dgc;
    }
  }
  lds_sync();
  // dgx_{r+1} into row r of Wg (its own element: one adder per element); the
  // norm's backward g_raw = f (g - x (x . g)) and the stores
#pragma unroll
  for (int j = 0; j < PPW; ++j) {
    const int pos = wave + 8 * j;
    if (pos < NPOS) {
      const int mt = pos / NT16, nt = pos % NT16, c = 16 * nt + li;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * mt + 4 * lg + e;
        if (r >= 1) Fm.Wg[r - 1][c] += dgx[j][e];
        if (!grouped && r < L) {
          float dq_dot = 0.f, dk_dot = 0.f;
#pragma unroll
          for (int u = 0; u < NT16; ++u) {
            dq_dot += Fm.nd[0][u][r];
            dk_dot += Fm.nd[1][u][r];
          }
          const float xq = l2norm ? sm.qh[r][c] / scale : 0.f, xk = l2norm ? sm.kh[r][c] : 0.f;
          const long o = ((tok0 + r) * Hk + hk) * DK + c;
          dq[o] = Fm.fq[r] * (oq[j][e] - xq * dq_dot);
          dk[o] = Fm.fk[r] * (ok[j][e] - xk * dk_dot);
        }
      }
    }
  }
  lds_sync();
  // dg_tc = sum_{r >= t} (dgam_rc + dgx_{r+1,c}) + dgC_c, from the last token up
  for (int c = tid; c < DK; c += kThr3) {
    float acc = sm.dgs[c] + Fm.dgcp[0][c] + Fm.dgcp[1][c];
    for (int t = kC - 1; t >= 0; --t) {
      acc += Fm.Wg[t][c];
      if (t < L) ddecay[((tok0 + t) * H + h) * DK + c] = acc;
    }
  }
  if (tid < kC && tid < L) {
    float db = sm.tb[tid];
#pragma unroll
    for (int nt = 0; nt < NT16; ++nt) db += Fm.dbp[nt][tid];
    dbeta[(tok0 + tid) * H + h] = db;
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
  // The reverse walk without per-channel decay fits two 16-column workgroups
  // per CU (its LDS): with more slices than that it takes 32 columns per
  // workgroup, so that every walk runs at once rather than in two rounds.
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 0;
  const bool wide = DV % 32 == 0 && cus > 0 && slices > 2u * static_cast<unsigned>(cus);
  if (a.decay_kind == DECAY_CHANNEL) {
    cbwd_prep_ch<DK, In><<<dim3(chunks), dim3(kThr), 0, s>>>(q, k, be, de, w, a.T, a.H, a.Hk, N, a.scale,
                                                              a.l2norm, a.tf);
    cbwd_fwd<DK, DV, In, true><<<dim3(slices), dim3(kThr), 0, s>>>(k, v, a.init, w, a.T, a.H, a.Hk, N, a.vfirst);
    cbwd_rev<DK, DV, In, true, kNS><<<dim3(slices), dim3(kThr), 0, s>>>(q, k, a.dout, a.dfinal, a.dv, a.dinit, w,
                                                                        a.T, a.H, a.Hk, N, a.vfirst);
    cbwd_local_ch<DK, DV, In><<<dim3(chunks), dim3(kThr3), 0, s>>>(q, k, v, a.dout, a.dq, a.dk, a.dbeta,
                                                                    a.ddecay, w, a.T, a.H, a.Hk, N, a.scale,
                                                                    a.l2norm);
    return hipGetLastError();
  }
  cbwd_prep<DK, In><<<dim3(chunks), dim3(kThr), 0, s>>>(q, k, be, de, a.decay_kind == DECAY_HEAD, w, a.T, a.H,
                                                         a.Hk, N, a.scale, a.l2norm, a.tf);
  cbwd_fwd<DK, DV, In, false><<<dim3(slices), dim3(kThr), 0, s>>>(k, v, a.init, w, a.T, a.H, a.Hk, N, a.vfirst);
  if (wide) {
    if constexpr (DV % 32 == 0)
      cbwd_rev<DK, DV, In, false, 32><<<dim3(slices / 2), dim3(kThr), 0, s>>>(q, k, a.dout, a.dfinal, a.dv, a.dinit,
                                                                              w, a.T, a.H, a.Hk, N, a.vfirst);
  } else {
    cbwd_rev<DK, DV, In, false, kNS><<<dim3(slices), dim3(kThr), 0, s>>>(q, k, a.dout, a.dfinal, a.dv, a.dinit, w,
                                                                         a.T, a.H, a.Hk, N, a.vfirst);
  }
  cbwd_local<DK, DV, In><<<dim3(chunks), dim3(kThr3), 0, s>>>(
      q, k, v, a.dout, a.dq, a.dk, a.dbeta, a.decay_kind == DECAY_HEAD ? a.ddecay : nullptr, w, a.T, a.H, a.Hk, N,
      a.scale, a.l2norm);
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
