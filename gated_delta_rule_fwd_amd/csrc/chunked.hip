// Fused chunked forward of the gated delta rule on gfx950.
//
// The recurrence (ejkernel kda, core recurrence) is computed "parallel within
// chunks, sequential across chunks" (ejkernel kda, Algorithm Modes) in the WY
// form the TileOPs DeltaNet pipeline names (prepare_wy_repr, then forward).
// For a chunk of C tokens entering with state S0 (DK x DV, rows = key
// channels), with G / Gx the inclusive / exclusive in-chunk cumulative log
// decay and sq, sk the query / key normalisers:
//
//   A  = strictly-lower  beta_r sk_r sk_s sum_c k_rc k_sc exp(Gx_rc - G_sc)
//   T  = (I + A)^-1                              (forward substitution in LDS)
//   W  = T diag(beta sk) (K * exp(Gx))          U = T diag(beta) V
//   D  = U - W S0                                (the per-token v_new)
//   O  = diag(sq) (Q * exp(G)) S0 + (lower-incl P) D,
//        P_rs = sq_r sk_s sum_c q_rc k_sc exp(G_rc - G_ss)
//   S  = exp(G_last) * S0 + (diag(sk) K * exp(G_last - G))^T D
//
// One workgroup owns one (batch, head, slice of DVS value columns) and walks
// all chunks of its sequence; the columns of S are independent, so the slice
// of S it owns lives in MFMA accumulators for the whole sequence and nothing
// but q, k, v, beta, decay (read) and o, final state (written) touches HBM.
// Each of the 4 waves owns 16 state columns; the WY work (A, T, W, P) is
// shared by the waves of the workgroup and recomputed by each slice.
//
// MFMA: v_mfma_f32_16x16x32_f16 for bf16 activations (raw bf16 values are
// exact in fp16; derived operands are rounded once to fp16) and
// v_mfma_f32_16x16x4_f32 for fp32 activations.  The inverse is built in fp32.
// Per-key-channel decay uses products of per-token factors exp(g) <= 1
// referenced to 16-token block boundaries, so that no factor exceeds 1 except
// the inverse-prefix operand of the diagonal blocks, which is kept in bf16
// (fp32 range); this needs the decay summed over any 16 consecutive tokens to
// stay above about -88 in every channel.
//
// Accumulator layout of a 16x16 MFMA result: lane l holds rows 4*(l/16)+j,
// j = 0..3, of column l%16.  The k index of an MFMA is a sum, so A and B may
// use any common permutation of it; the kernel uses k = 4*(l/16)+j within each
// 16-wide k block, which lets an accumulator tile be fed back as the B operand
// (or, read transposed, as the A operand) of the next product without an LDS
// round trip.
#include "chunked_layout.h"
#include "common.h"
#include "launch.h"

namespace kda {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr float kSafeBlockDecay = 1.1253517e-07f;   // exp(-16)

// ---------------------------------------------------------------- MFMA ops --

template <typename OpT> struct Mma;

template <> struct Mma<_Float16> {
  using T = _Float16;
  using frag = f16x8;
  // k = k0 + 8*g + e  (e = 0..7)
  __device__ static frag ld_cont(const T* row, int k0, int g) {
    return *reinterpret_cast<const f16x8*>(row + k0 + 8 * g);
  }
  // k = k0 + 4*g + e (e < 4) and k0 + 16 + 4*g + e - 4 (e >= 4)
  __device__ static frag ld_perm(const T* row, int k0, int g) {
    const f16x4 lo = *reinterpret_cast<const f16x4*>(row + k0 + 4 * g);
    const f16x4 hi = *reinterpret_cast<const f16x4*>(row + k0 + 16 + 4 * g);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  __device__ static frag from_acc(const f32x4& a, const f32x4& b) {
    frag f;
    f[0] = (T)a[0]; f[1] = (T)a[1]; f[2] = (T)a[2]; f[3] = (T)a[3];
    f[4] = (T)b[0]; f[5] = (T)b[1]; f[6] = (T)b[2]; f[7] = (T)b[3];
    return f;
  }
  __device__ static frag zero() { return frag{0, 0, 0, 0, 0, 0, 0, 0}; }
  __device__ static void mma(f32x4& acc, const frag& a, const frag& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc, 0, 0, 0);
  }
  __device__ static void store4(T* p, const f32x4& v) {
    f16x4 h;
    h[0] = (T)v[0]; h[1] = (T)v[1]; h[2] = (T)v[2]; h[3] = (T)v[3];
    *reinterpret_cast<f16x4*>(p) = h;
  }
};

template <> struct Mma<float> {
  using T = float;
  struct frag { f32x4 lo, hi; };
  // fp32 MFMA takes one k per lane per instruction; four instructions cover a
  // 16-wide k block with k = 4*g + j, so "cont" and "perm" are the same map.
  __device__ static frag ld_perm(const T* row, int k0, int g) {
    frag f;
    f.lo = *reinterpret_cast<const f32x4*>(row + k0 + 4 * g);
    f.hi = *reinterpret_cast<const f32x4*>(row + k0 + 16 + 4 * g);
    return f;
  }
  __device__ static frag ld_cont(const T* row, int k0, int g) { return ld_perm(row, k0, g); }
  __device__ static frag from_acc(const f32x4& a, const f32x4& b) { return frag{a, b}; }
  __device__ static frag zero() { return frag{f32x4{0, 0, 0, 0}, f32x4{0, 0, 0, 0}}; }
  __device__ static void mma(f32x4& acc, const frag& a, const frag& b) {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[j], b.lo[j], acc, 0, 0, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[j], b.hi[j], acc, 0, 0, 0);
  }
  __device__ static void store4(T* p, const f32x4& v) { *reinterpret_cast<f32x4*>(p) = v; }
};

// Diagonal-block Gram of the per-channel path: bf16 x bf16 (fp32 exponent range)
// for bf16 activations, plain fp32 for fp32 activations.
__device__ __forceinline__ void mma_diag(f32x4& acc, const f16x8& a_f16, const uint16_t* kinv_row,
                                         int k0, int g) {
  // Whole-vector bit casts: building a __bf16 vector element by element from
  // 16-bit patterns is not reliably compiled.
  const uint4 braw = *reinterpret_cast<const uint4*>(kinv_row + k0 + 8 * g);
  uint32_t aw[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t lo = f32_to_bf16(static_cast<float>(a_f16[2 * e]));
    const uint32_t hi = f32_to_bf16(static_cast<float>(a_f16[2 * e + 1]));
    aw[e] = lo | (hi << 16);
  }
  const uint4 araw = uint4{aw[0], aw[1], aw[2], aw[3]};
  const bf16x8 a = __builtin_bit_cast(bf16x8, araw);
  const bf16x8 b = __builtin_bit_cast(bf16x8, braw);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}

template <typename In> struct OpOf { using T = _Float16; using KinvT = uint16_t; };
template <> struct OpOf<float> { using T = float; using KinvT = float; };

__device__ __forceinline__ void put_kinv(uint16_t* p, float x) { *p = f32_to_bf16(x); }
__device__ __forceinline__ void put_kinv(float* p, float x) { *p = x; }

struct ChunkParams {
  const void* q; const void* k; const void* v; const void* beta; const void* decay;
  const float* init; float* o; float* state;
  int T, H, DV, C, nsl, xcd_map, decay_kind, l2norm;
  float scale;
};

// ------------------------------------------------------------------ kernel --

template <int DK, int DVS, int CM, typename In>
__global__ __launch_bounds__(kThreads, 1) void chunked_kernel(ChunkParams p) {
  using OpT = typename OpOf<In>::T;
  using KinvT = typename OpOf<In>::KinvT;
  using M = Mma<OpT>;
  using L = ChunkLayout<DK, DVS, CM, sizeof(OpT)>;
  constexpr int V = act<In>::kVec;          // activation elements per 16-byte load
  constexpr int LPR = DK / V;               // lanes per q/k row
  constexpr int RPP = kThreads / LPR;       // q/k rows per load pass
  constexpr int NP = (CM + RPP - 1) / RPP;  // q/k load passes
  constexpr int LPRv = DVS / V;
  constexpr int RPPv = kThreads / LPRv;
  constexpr int NPv = (CM + RPPv - 1) / RPPv;
  constexpr int NBM = CM / 16;              // row blocks at the largest chunk
  constexpr int NKT = DK / 16;              // 16-row state tiles
  constexpr int NKP = DK / 32;              // 32-wide k steps over the key dim
  static_assert(LPR <= 64 && (64 % LPR) == 0, "q/k rows must pack into waves");
  static_assert(LPRv >= 1 && (64 % LPRv) == 0, "v rows must pack into waves");
  static_assert(DVS % 16 == 0 && DVS <= 16 * kWaves, "slice width");

  extern __shared__ __align__(256) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int T = p.T, H = p.H, DV = p.DV, C = p.C;
  const int nb = C / 16;
  const int decay_kind = p.decay_kind;
  const bool chan = decay_kind == DECAY_CHANNEL;
  const bool headdecay = decay_kind == DECAY_HEAD;

  // Workgroup -> (head, slice).  With xcd_map the slices of one head get ids
  // that are equal mod 8, i.e. run on the same XCD and share its L2.
  int head, slice;
  {
    const int id = blockIdx.x;
    if (p.xcd_map) {
      const int x = id & 7, qd = id >> 3;
      head = (qd / p.nsl) * 8 + x;
      slice = qd % p.nsl;
    } else {
      head = id / p.nsl;
      slice = id % p.nsl;
    }
  }
  const int b = head / H, h = head % H;
  const int n0 = slice * DVS;   // first value column of this slice

  OpT* sQ = reinterpret_cast<OpT*>(smem + L::oQ);
  OpT* sKT = reinterpret_cast<OpT*>(smem + L::oKT);
  OpT* sVT = reinterpret_cast<OpT*>(smem + L::oVT);
  OpT* sP = reinterpret_cast<OpT*>(smem + L::oP);
  OpT* sK = reinterpret_cast<OpT*>(smem + L::oRA);
  float* sTm = reinterpret_cast<float*>(smem + L::oRA);
  float* sAm = reinterpret_cast<float*>(smem + L::oRB);
  OpT* sWn = reinterpret_cast<OpT*>(smem + L::oRB);
  OpT* sKb = reinterpret_cast<OpT*>(smem + L::oRC);
  KinvT* sKinv = reinterpret_cast<KinvT*>(smem + L::oRC + L::kRowTile);
  OpT* sTw = reinterpret_cast<OpT*>(smem + L::oRC);
  OpT* sTu = reinterpret_cast<OpT*>(smem + L::oRC + L::kCC);
  OpT* sKF = reinterpret_cast<OpT*>(smem + L::oKF(true));
  OpT* sGst = sKF;   // staged per-channel gate, [CM][DK]
  float* sv = reinterpret_cast<float*>(smem + L::oVec(chan));
  float* s_bt = sv + 2 * CM;
  float* s_Gi = sv + 3 * CM;
  float* s_Ge = sv + 4 * CM;
  float* s_eG = sv + 5 * CM;
  float* s_eGx = sv + 6 * CM;
  float* s_eF = sv + 7 * CM;
  float* s_misc = sv + 8 * CM;                 // [0] = exp(G_last), [1] = unsafe-gate flag
  int* s_flag = reinterpret_cast<int*>(s_misc + 1);
  float* s_tau = s_misc + 16;                  // [NBM][DK] whole-block decay factors
  float* s_Cb = s_tau + NBM * DK;              // [NBM][DK] decay of all earlier blocks
  float* s_rsq = s_Cb + NBM * DK;              // [NBM][DK] 1/sqrt(block factor)
  float* s_D = s_rsq + NBM * DK;               // [ND][DK] decay of blocks strictly between i, j
  float* s_decC = s_D + L::ND * DK;            // [DK] decay of the whole chunk

  // Zero all of LDS once: padding columns and never-written upper blocks must
  // read as zero in every chunk.
  {
    const int nvec = static_cast<int>(L::bytes(chan) / 16);
    uint4* z = reinterpret_cast<uint4*>(smem);
    for (int i = tid; i < nvec; i += kThreads) z[i] = uint4{0, 0, 0, 0};
  }

  const In* gq = static_cast<const In*>(p.q);
  const In* gk = static_cast<const In*>(p.k);
  const In* gv = static_cast<const In*>(p.v);
  const In* gb = static_cast<const In*>(p.beta);
  const In* gg = static_cast<const In*>(p.decay);
  const long tok0 = static_cast<long>(b) * T;   // token index base of this sequence

  // ---- prefetch registers (one chunk ahead) ----
  uint4 rq[NP], rk[NP], rg[NP], rv[NPv];
  float rbeta = 0.f, rgh = 0.f;

  auto issue_loads = [&](int t0) {
    const int Lc = min(C, T - t0);
#pragma unroll
    for (int pp = 0; pp < NP; ++pp) {
      const int r = pp * RPP + tid / LPR, seg = tid % LPR;
      rq[pp] = rk[pp] = rg[pp] = uint4{0, 0, 0, 0};
      if (r < Lc) {
        const long off = ((tok0 + t0 + r) * H + h) * DK + seg * V;
        rq[pp] = *reinterpret_cast<const uint4*>(gq + off);
        rk[pp] = *reinterpret_cast<const uint4*>(gk + off);
        if (chan) rg[pp] = *reinterpret_cast<const uint4*>(gg + off);
      }
    }
#pragma unroll
    for (int pp = 0; pp < NPv; ++pp) {
      const int r = pp * RPPv + tid / LPRv, seg = tid % LPRv;
      rv[pp] = uint4{0, 0, 0, 0};
      if (r < Lc) {
        const long off = ((tok0 + t0 + r) * H + h) * static_cast<long>(DV) + n0 + seg * V;
        rv[pp] = *reinterpret_cast<const uint4*>(gv + off);
      }
    }
    rbeta = 0.f; rgh = 0.f;
    if (tid < CM && tid < Lc) {
      const long off = (tok0 + t0 + tid) * H + h;
      rbeta = act<In>::load1(gb + off);
      if (headdecay) rgh = act<In>::load1(gg + off);
    }
  };
  auto unpack = [&](const uint4& raw, float (&x)[V]) {
    act<In>::load_vec(reinterpret_cast<const In*>(&raw), x);
  };

  // ---- the state slice: wave w owns value columns n0 + 16w .. +15 ----
  const bool owner = wave < DVS / 16;
  const int ncol = n0 + 16 * wave + l16;   // this lane's value column (owner waves)
  f32x4 S[NKT];
#pragma unroll
  for (int t = 0; t < NKT; ++t) {
    S[t] = f32x4{0, 0, 0, 0};
    if (owner && p.init) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        S[t][j] = p.init[((static_cast<long>(b) * H + h) * DK + 16 * t + 4 * g + j) * DV + ncol];
    }
  }

  const int nchunks = (T + C - 1) / C;
  if (nchunks > 0) issue_loads(0);
  __syncthreads();   // LDS zero-fill visible

  for (int ch = 0; ch < nchunks; ++ch) {
    const int t0 = ch * C;
    const int Lc = min(C, T - t0);

    // ================= phase 1: stage the chunk, norms, gates =================
#pragma unroll
    for (int pp = 0; pp < NP; ++pp) {
      const int r = pp * RPP + tid / LPR, seg = tid % LPR;
      float qv[V], kv[V];
      unpack(rq[pp], qv);
      unpack(rk[pp], kv);
      float sq = 0.f, sk = 0.f;
#pragma unroll
      for (int e = 0; e < V; ++e) { sq += qv[e] * qv[e]; sk += kv[e] * kv[e]; }
      sq = group_sum<LPR>(sq);
      sk = group_sum<LPR>(sk);
      // normalised (and, for q, scaled) rows: |k_hat| <= 1 keeps every fp16
      // operand far from overflow whatever the raw magnitudes
      const float qn = (p.l2norm ? inv_norm(sq) : 1.f) * p.scale;
      const float kn = p.l2norm ? inv_norm(sk) : 1.f;
#pragma unroll
      for (int e = 0; e < V; ++e) { qv[e] *= qn; kv[e] *= kn; }
      if (r < CM) {
        OpT* qrow = sQ + r * L::LDK + seg * V;
        OpT* krow = sK + r * L::LDK + seg * V;
#pragma unroll
        for (int e = 0; e < V; ++e) { qrow[e] = (OpT)qv[e]; krow[e] = (OpT)kv[e]; }
        if (!chan) {
#pragma unroll
          for (int e = 0; e < V; ++e) sKT[(seg * V + e) * L::LC + r] = (OpT)kv[e];
        } else {
          float gvv[V];
          unpack(rg[pp], gvv);
          OpT* grow = sGst + r * DK + seg * V;
#pragma unroll
          for (int e = 0; e < V; ++e) grow[e] = (OpT)gvv[e];
        }
      }
    }
#pragma unroll
    for (int pp = 0; pp < NPv; ++pp) {
      const int r = pp * RPPv + tid / LPRv, seg = tid % LPRv;
      if (r < CM) {
        float vv[V];
        unpack(rv[pp], vv);
#pragma unroll
        for (int e = 0; e < V; ++e) sVT[(seg * V + e) * L::LC + r] = (OpT)vv[e];
      }
    }
    if (wave == 0) {
      // beta and the scalar gate: lane r holds token r of the chunk (CM <= 64).
      const float gr = (tid < CM) ? rgh : 0.f;
      float G = gr;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(G, off, 64);
        if (lane >= off) G += y;
      }
      float Gx = __shfl_up(G, 1, 64);
      if (lane == 0) Gx = 0.f;
      const float Glast = __shfl(G, 63, 64);
      if (lane < CM) {
        s_bt[lane] = rbeta;
        s_Gi[lane] = G;
        s_Ge[lane] = Gx;
        s_eG[lane] = __expf(G);
        s_eGx[lane] = __expf(Gx);
        s_eF[lane] = __expf(Glast - G);
      }
      if (lane == 0) {
        s_misc[0] = __expf(Glast);
        *s_flag = 0;
      }
    }
    // registers are free: fetch the next chunk while this one is computed
    if (ch + 1 < nchunks) issue_loads(t0 + C);
    __syncthreads();

    if (chan) {
      // (1b) per (16-token block, key channel): exp(g) products referenced to
      // the block start (prefix) and end (suffix); all of them are <= 1.
      constexpr int NT = (NBM * DK + kThreads - 1) / kThreads;
      // bf16 fallback copy of the inverse-prefix operand, two values per register
      uint32_t kin16[NT][8];
#pragma unroll
      for (int it = 0; it < NT; ++it) {
        const int task = tid + it * kThreads;
        if (task < NBM * DK) {
          const int i = task / DK, c = task % DK;
          float a[16], kx[16], kin[16];
          float pre = 1.f;
#pragma unroll
          for (int t = 0; t < 16; ++t) {
            const int r = 16 * i + t;
            a[t] = __expf(static_cast<float>(sGst[r * DK + c]));
            kx[t] = static_cast<float>(sK[r * L::LDK + c]);
            const float qx = static_cast<float>(sQ[r * L::LDK + c]);
            sK[r * L::LDK + c] = (OpT)(kx[t] * pre);          // Ka: exclusive prefix
            pre *= a[t];
            kin[t] = kx[t] / pre;                             // k / inclusive prefix
            sQ[r * L::LDK + c] = (OpT)(qx * pre);             // Qa: inclusive prefix
          }
          float suf = 1.f;
#pragma unroll
          for (int t = 15; t >= 0; --t) {
            sKb[(16 * i + t) * L::LDK + c] = (OpT)(kx[t] * suf);  // Kb: decay to block end
            suf *= a[t];
          }
          s_tau[i * DK + c] = pre;   // whole-block factor
          if constexpr (sizeof(OpT) == 2) {
            // The diagonal blocks pair a factor <= 1 with its inverse.  Balanced
            // by sqrt(block factor), both stay within exp(+-8) when the block
            // decays by at most exp(-16), which fp16 holds; otherwise the chunk
            // falls back to a bf16 (fp32-range) inverse-prefix operand.
            const float rs = sqrtf(pre);
            s_rsq[i * DK + c] = 1.f / rs;
#pragma unroll
            for (int t = 0; t < 16; ++t) {
              *reinterpret_cast<_Float16*>(&sKinv[(16 * i + t) * L::LDK + c]) = (_Float16)(kin[t] * rs);
            }
#pragma unroll
            for (int t = 0; t < 8; ++t)
              kin16[it][t] = static_cast<uint32_t>(f32_to_bf16(kin[2 * t])) |
                             (static_cast<uint32_t>(f32_to_bf16(kin[2 * t + 1])) << 16);
            if (pre < kSafeBlockDecay) *s_flag = 1;
          } else {
#pragma unroll
            for (int t = 0; t < 16; ++t) put_kinv(&sKinv[(16 * i + t) * L::LDK + c], kin[t]);
          }
        }
      }
      __syncthreads();
      const bool safe = *s_flag == 0;
      // (1c) chunk-level factors: transposed operands for W and the state
      // update; the bf16 inverse-prefix operand where fp16 range is short.
#pragma unroll
      for (int it = 0; it < NT; ++it) {
        const int task = tid + it * kThreads;
        if (task < NBM * DK) {
          const int i = task / DK, c = task % DK;
          const float tau = s_tau[i * DK + c];
          if constexpr (sizeof(OpT) == 2) {
            if (!safe) {
#pragma unroll
              for (int t = 0; t < 16; ++t)
                sKinv[(16 * i + t) * L::LDK + c] = static_cast<uint16_t>(kin16[it][t >> 1] >> (16 * (t & 1)));
            }
          }
          float cb = 1.f, ca = 1.f;
          for (int j = 0; j < i; ++j) cb *= s_tau[j * DK + c];
          for (int j = i + 1; j < NBM; ++j) ca *= s_tau[j * DK + c];
          s_Cb[i * DK + c] = cb;
          if (i == 0) s_decC[c] = ca * tau;
          float dd = 1.f;
          for (int j = i - 1; j >= 0; --j) {    // D[i][j] = prod_{j < m < i} tau_m
            if (i - j >= 2) s_D[L::dslot(i, j) * DK + c] = dd;
            dd *= s_tau[j * DK + c];
          }
          OpT* ket = sKT + c * L::LC + 16 * i;
          OpT* kft = sKF + c * L::LC + 16 * i;
#pragma unroll
          for (int t = 0; t < 16; ++t) {
            const int r = 16 * i + t;
            ket[t] = (OpT)(static_cast<float>(sK[r * L::LDK + c]) * cb);
            kft[t] = (OpT)(static_cast<float>(sKb[r * L::LDK + c]) * ca);
          }
        }
      }
      __syncthreads();
    }

    // ================= phase 2: Gram A (strict) and P (inclusive) =================
    {
      const int npairs = nb * (nb + 1) / 2;
      for (int job = wave; job < 2 * npairs; job += kWaves) {
        const bool isP = job >= npairs;
        int pi = isP ? job - npairs : job;
        int i = 0;
        while (pi > i) { pi -= i + 1; ++i; }
        const int j = pi;
        const OpT* arow = (isP ? sQ : sK) + (16 * i + l16) * L::LDK;
        const OpT* brow = (chan ? sKb : sK) + (16 * j + l16) * L::LDK;
        f32x4 acc = {0, 0, 0, 0};
        if (chan && i == j) {
          if constexpr (sizeof(OpT) == 2) {
            const KinvT* krow = sKinv + (16 * j + l16) * L::LDK;
            if (*s_flag == 0) {
              const OpT* krh = reinterpret_cast<const OpT*>(krow);
              const float* rsq = s_rsq + i * DK;
#pragma unroll
              for (int m = 0; m < NKP; ++m) {
                auto fa = M::ld_cont(arow, 32 * m, g);
#pragma unroll
                for (int e = 0; e < 8; ++e) fa[e] = (OpT)(static_cast<float>(fa[e]) * rsq[32 * m + 8 * g + e]);
                M::mma(acc, fa, M::ld_cont(krh, 32 * m, g));
              }
            } else {
#pragma unroll
              for (int m = 0; m < NKP; ++m) mma_diag(acc, M::ld_cont(arow, 32 * m, g), krow, 32 * m, g);
            }
          } else {
            const OpT* krow = reinterpret_cast<const OpT*>(sKinv) + (16 * j + l16) * L::LDK;
#pragma unroll
            for (int m = 0; m < NKP; ++m) M::mma(acc, M::ld_cont(arow, 32 * m, g), M::ld_cont(krow, 32 * m, g));
          }
        } else if (chan && i - j >= 2) {
          const float* dv = s_D + L::dslot(i, j) * DK;
#pragma unroll
          for (int m = 0; m < NKP; ++m) {
            auto fa = M::ld_cont(arow, 32 * m, g);
            if constexpr (sizeof(OpT) == 2) {
#pragma unroll
              for (int e = 0; e < 8; ++e) fa[e] = (OpT)(static_cast<float>(fa[e]) * dv[32 * m + 8 * g + e]);
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                fa.lo[e] *= dv[32 * m + 4 * g + e];
                fa.hi[e] *= dv[32 * m + 16 + 4 * g + e];
              }
            }
            M::mma(acc, fa, M::ld_cont(brow, 32 * m, g));
          }
        } else {
#pragma unroll
          for (int m = 0; m < NKP; ++m) M::mma(acc, M::ld_cont(arow, 32 * m, g), M::ld_cont(brow, 32 * m, g));
        }
        const int s = 16 * j + l16;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int r = 16 * i + 4 * g + jj;
          if (!isP) {
            float f = s_bt[r];
            if (headdecay) f *= __expf(s_Ge[r] - s_Gi[s]);
            const float val = acc[jj] * f;
            sAm[r * L::LF + s] = (s < r) ? val : 0.f;
          } else {
            float val = acc[jj];
            if (headdecay) val *= __expf(s_Gi[r] - s_Gi[s]);
            sP[r * L::LC + s] = (OpT)((s <= r) ? val : 0.f);
          }
        }
      }
    }
    __syncthreads();

    // ================= phase 3: T = (I + A)^-1 =================
    if (wave == 0) {
      // diagonal 16x16 blocks: lane -> (block, column), forward substitution
      const int i = g, jc = l16;
      if (i < nb) {
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float* arow = sAm + (16 * i + r) * L::LF + 16 * i;
          float acc = (r == jc) ? 1.f : 0.f;
#pragma unroll
          for (int s = 0; s < r; ++s) acc -= arow[s] * x[s];
          x[r] = acc;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) sTm[(16 * i + r) * L::LF + 16 * i + jc] = x[r];
      }
    } else if (chan) {
      // decayed query for the output: Q * exp(G) = Qa * (product of earlier blocks)
      for (int idx = tid - 64; idx < nb * 16 * DK; idx += kThreads - 64) {
        const int r = idx / DK, c = idx % DK;
        OpT* qp = sQ + r * L::LDK + c;
        *qp = (OpT)(static_cast<float>(*qp) * s_Cb[(r >> 4) * DK + c]);
      }
    }
    __syncthreads();
    for (int d = 1; d < nb; ++d) {
      // off-diagonal blocks on diagonal d: T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj
      const int j = wave, i = wave + d;
      if (i < nb) {
        f32x4 X = {0, 0, 0, 0};
        for (int kb = j; kb < i; ++kb) {
          const f32x4 a4 = *reinterpret_cast<const f32x4*>(sAm + (16 * i + l16) * L::LF + 16 * kb + 4 * g);
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const float bv = sTm[(16 * kb + 4 * g + jj) * L::LF + 16 * j + l16];
            X = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[jj], bv, X, 0, 0, 0);
          }
        }
        const f32x4 t4 = *reinterpret_cast<const f32x4*>(sTm + (16 * i + l16) * L::LF + 16 * i + 4 * g);
        f32x4 Y = {0, 0, 0, 0};
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) Y = __builtin_amdgcn_mfma_f32_16x16x4f32(t4[jj], X[jj], Y, 0, 0, 0);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) sTm[(16 * i + 4 * g + jj) * L::LF + 16 * j + l16] = -Y[jj];
      }
      __syncthreads();
    }
    // Tw = T diag(beta sk [exp(Gx)]),  Tu = T diag(beta); zero above the block diagonal
    {
      const int ncols = (nb + 1) / 2 * 32;   // k range read by the 32-wide steps
      for (int idx = tid; idx < nb * 16 * ncols; idx += kThreads) {
        const int r = idx / ncols, s = idx % ncols;
        float t = 0.f;
        if (s < C && (s >> 4) <= (r >> 4)) t = sTm[r * L::LF + s];
        float cw = 0.f, cu = 0.f;
        if (s < CM) {
          cu = s_bt[s];
          cw = headdecay ? cu * s_eGx[s] : cu;
        }
        sTw[r * L::LC + s] = (OpT)(t * cw);
        sTu[r * L::LC + s] = (OpT)(t * cu);
      }
    }
    __syncthreads();

    // ================= phase 4: -W (W^T = KX Tw^T) =================
    for (int job = wave; job < NKT * nb; job += kWaves) {
      const int ct = job % NKT, rt = job / NKT;
      const OpT* arow = sKT + (16 * ct + l16) * L::LC;
      const OpT* brow = sTw + (16 * rt + l16) * L::LC;
      f32x4 acc = {0, 0, 0, 0};
      for (int m = 0; m <= rt / 2; ++m) M::mma(acc, M::ld_cont(arow, 32 * m, g), M::ld_cont(brow, 32 * m, g));
      M::store4(sWn + (16 * rt + l16) * L::LDK + 16 * ct + 4 * g, -acc);
    }
    __syncthreads();

    // ================= phase 5: state step and output (per owner wave) =================
    if (owner) {
      const OpT* vrow = sVT + (16 * wave + l16) * L::LC;
      f32x4 Dl[NBM];
#pragma unroll
      for (int rt = 0; rt < NBM; ++rt) {
        Dl[rt] = f32x4{0, 0, 0, 0};
        if (rt < nb) {
          const OpT* urow = sTu + (16 * rt + l16) * L::LC;
          for (int m = 0; m <= rt / 2; ++m) M::mma(Dl[rt], M::ld_cont(urow, 32 * m, g), M::ld_cont(vrow, 32 * m, g));
        }
      }
      typename M::frag Sf[NKP];
#pragma unroll
      for (int m = 0; m < NKP; ++m) Sf[m] = M::from_acc(S[2 * m], S[2 * m + 1]);
      // D = U - W S0
#pragma unroll
      for (int rt = 0; rt < NBM; ++rt) {
        if (rt < nb) {
          const OpT* wrow = sWn + (16 * rt + l16) * L::LDK;
#pragma unroll
          for (int m = 0; m < NKP; ++m) M::mma(Dl[rt], M::ld_perm(wrow, 32 * m, g), Sf[m]);
        }
      }
      typename M::frag Df[NBM / 2];
#pragma unroll
      for (int m = 0; m < NBM / 2; ++m) Df[m] = M::from_acc(Dl[2 * m], Dl[2 * m + 1]);
      // O^T = S0^T (scaled Q)^T + D^T P^T, one 16-token tile at a time
#pragma unroll
      for (int rt = 0; rt < NBM; ++rt) {
        if (rt < nb) {
          const OpT* qrow = sQ + (16 * rt + l16) * L::LDK;
          f32x4 acc = {0, 0, 0, 0};
#pragma unroll
          for (int m = 0; m < NKP; ++m) M::mma(acc, Sf[m], M::ld_perm(qrow, 32 * m, g));
          const int r = 16 * rt + l16;
          if (headdecay) acc *= s_eG[r];
          const OpT* prow = sP + r * L::LC;
          for (int m = 0; m <= rt / 2; ++m) M::mma(acc, Df[m], M::ld_perm(prow, 32 * m, g));
          if (r < Lc) {
            float* op = p.o + ((tok0 + t0 + r) * H + h) * static_cast<long>(DV) + n0 + 16 * wave + 4 * g;
            *reinterpret_cast<f32x4*>(op) = acc;
          }
        }
      }
      // S <- exp(G_last) S0 + KY D'
      const float eGC = headdecay ? s_misc[0] : 1.f;
#pragma unroll
      for (int t = 0; t < NKT; ++t) {
        if (chan) {
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) S[t][jj] *= s_decC[16 * t + 4 * g + jj];
        } else {
          S[t] *= eGC;
        }
      }
      if (headdecay) {
#pragma unroll
        for (int st = 0; st < NBM; ++st) {
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) Dl[st][jj] *= s_eF[16 * st + 4 * g + jj];
        }
      }
#pragma unroll
      for (int m = 0; m < NBM / 2; ++m) Df[m] = M::from_acc(Dl[2 * m], Dl[2 * m + 1]);
      const OpT* KY = chan ? sKF : sKT;
      const int nkm = (nb + 1) / 2;
#pragma unroll
      for (int t = 0; t < NKT; ++t) {
        const OpT* arow = KY + (16 * t + l16) * L::LC;
        for (int m = 0; m < nkm; ++m) M::mma(S[t], M::ld_perm(arow, 32 * m, g), Df[m]);
      }
    }
    __syncthreads();
  }

  if (owner) {
#pragma unroll
    for (int t = 0; t < NKT; ++t) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        p.state[((static_cast<long>(b) * H + h) * DK + 16 * t + 4 * g + j) * DV + ncol] = S[t][j];
    }
  }
}

// ---------------------------------------------------------------- launcher --

template <int DK, int DVS, int CM, typename In>
hipError_t launch_one(const ChunkParams& cp, int nwg, bool chan, hipStream_t s) {
  using OpT = typename OpOf<In>::T;
  using L = ChunkLayout<DK, DVS, CM, sizeof(OpT)>;
  const size_t lds = L::bytes(chan);
  if (lds > kMaxLds) return hipErrorInvalidConfiguration;
  auto fn = chunked_kernel<DK, DVS, CM, In>;
  static bool attr_set = false;   // benign race: the attribute call is idempotent
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(kMaxLds));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  fn<<<dim3(nwg), dim3(kThreads), lds, s>>>(cp);
  return hipGetLastError();
}

template <int DK, int CM, typename In>
hipError_t by_dvs(int dvs, const ChunkParams& cp, int nwg, bool chan, hipStream_t s) {
  switch (dvs) {
    case 16: return launch_one<DK, 16, CM, In>(cp, nwg, chan, s);
    case 32: return launch_one<DK, 32, CM, In>(cp, nwg, chan, s);
    case 64: return launch_one<DK, 64, CM, In>(cp, nwg, chan, s);
  }
  return hipErrorInvalidValue;
}

template <typename In, int CM>
hipError_t by_dk(int dk, int dvs, const ChunkParams& cp, int nwg, bool chan, hipStream_t s) {
  switch (dk) {
    case 32: return by_dvs<32, CM, In>(dvs, cp, nwg, chan, s);
    case 64: return by_dvs<64, CM, In>(dvs, cp, nwg, chan, s);
    case 128: return by_dvs<128, CM, In>(dvs, cp, nwg, chan, s);
  }
  return hipErrorInvalidValue;
}

template <int DK, int DVS, int CM, int OpBytes>
constexpr size_t lds_of(bool chan) { return ChunkLayout<DK, DVS, CM, OpBytes>::bytes(chan); }

size_t lds_for(int DK, int DVS, int CM, int opbytes, bool chan) {
#define KDA_L(dk, dvs, cm, ob) \
  if (DK == dk && DVS == dvs && CM == cm && opbytes == ob) return lds_of<dk, dvs, cm, ob>(chan);
#define KDA_L2(dk, cm, ob) KDA_L(dk, 16, cm, ob) KDA_L(dk, 32, cm, ob) KDA_L(dk, 64, cm, ob)
#define KDA_L3(cm, ob) KDA_L2(32, cm, ob) KDA_L2(64, cm, ob) KDA_L2(128, cm, ob)
  KDA_L3(64, 2) KDA_L3(32, 4) KDA_L3(64, 4)
#undef KDA_L3
#undef KDA_L2
#undef KDA_L
  return 0;
}

// Pick the value-slice width: enough workgroups to cover the 256 CUs, no
// wider than 64 columns, and an LDS plan that fits.
struct Plan { int dvs, cm; size_t lds; };

Plan plan_for(int B, int H, int DK, int DV, int C, int dtype, bool chan) {
  const int opb = dtype == 0 ? 4 : 2;
  const int cm = dtype == 0 ? (C <= 32 ? 32 : 64) : 64;
  int dvs = DV < 64 ? DV : 64;
  while (dvs > 16 && static_cast<long>(B) * H * (DV / dvs) < 256) dvs /= 2;
  while (dvs >= 16) {
    const size_t l = lds_for(DK, dvs, cm, opb, chan);
    if (l != 0 && l <= kMaxLds) return Plan{dvs, cm, l};
    dvs /= 2;
  }
  return Plan{0, cm, 0};
}

}  // namespace

size_t chunked_lds_bytes(int DK, int DV, int chunk, int dtype) {
  // worst case over decay kinds at the smallest grid (B = H = 1)
  const Plan a = plan_for(1, 1, DK, DV, chunk, dtype, true);
  const Plan b = plan_for(1, 1, DK, DV, chunk, dtype, false);
  if (a.dvs == 0 || b.dvs == 0) return 0;
  return a.lds > b.lds ? a.lds : b.lds;
}

hipError_t launch_chunked(const FwdArgs& a, hipStream_t s) {
  const bool chan = a.decay_kind == DECAY_CHANNEL;
  const Plan pl = plan_for(a.B, a.H, a.DK, a.DV, a.chunk, a.dtype, chan);
  if (pl.dvs == 0) return hipErrorInvalidConfiguration;
  ChunkParams cp;
  cp.q = a.q; cp.k = a.k; cp.v = a.v; cp.beta = a.beta; cp.decay = a.decay;
  cp.init = a.init; cp.o = a.o; cp.state = a.state;
  cp.T = a.T; cp.H = a.H; cp.DV = a.DV; cp.C = a.chunk;
  cp.nsl = a.DV / pl.dvs;
  cp.decay_kind = a.decay_kind;
  cp.l2norm = a.l2norm;
  cp.scale = a.scale;
  const int nheads = a.B * a.H;
  cp.xcd_map = (nheads % 8 == 0) ? 1 : 0;
  const int nwg = nheads * cp.nsl;
  if (a.dtype == 0) {
    return pl.cm == 32 ? by_dk<float, 32>(a.DK, pl.dvs, cp, nwg, chan, s)
                       : by_dk<float, 64>(a.DK, pl.dvs, cp, nwg, chan, s);
  }
  return by_dk<bf16_t, 64>(a.DK, pl.dvs, cp, nwg, chan, s);
}

}  // namespace kda
