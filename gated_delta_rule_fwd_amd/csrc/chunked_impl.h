// Fused chunked forward of the gated delta rule on gfx950 (kernel template).
//
// The recurrence (ejkernel kda, core recurrence) is computed "parallel within
// chunks, sequential across chunks" (ejkernel kda, Algorithm Modes) in the WY
// form the TileOPs DeltaNet pipeline names (prepare_wy_repr, then forward).
// For a chunk of C tokens entering with state S0 (DK x DV, rows = key
// channels), with normalised k_hat, scaled normalised q_hat, and G / Gx the
// inclusive / exclusive in-chunk cumulative log decay per key channel:
//
//   A  = strictly lower: A_rs = beta_r sum_c k_rc k_sc exp(Gx_rc - G_sc)
//   T  = (I + A)^-1                               (blocked substitution in LDS)
//   D  = T diag(beta) (V - (K * exp(Gx)) S0)      (the per-token v_new)
//   O  = (Q * exp(G)) S0 + (lower-inclusive P) D,  P_rs = sum_c q_rc k_sc exp(G_rc - G_sc)
//   S  = exp(G_last) * S0 + (K * exp(G_last - G))^T D
//
// (D is the WY form U - W S0 with U = T diag(beta) V and W = T diag(beta)
// (K * exp(Gx)), associated so that W is never formed.)
//
// One workgroup owns one (batch, head, slice of DVS value columns) and walks
// all chunks of its sequence.  The columns of S are independent, so each of
// its DVS/16 "owner" waves keeps 16 columns of S in MFMA accumulators for the
// whole sequence; the chunk-shared work (normalisation, gates, A, P, T) is
// spread over all 4 waves and recomputed by every slice of a head.  Only
// q, k, v, beta, decay (read once) and o, the final state (written once)
// touch HBM.
//
// MFMA: v_mfma_f32_16x16x32_f16 for bf16 activations (q, k normalised and v
// rounded once to fp16; derived operands rounded once to fp16) and
// v_mfma_f32_16x16x4_f32 for fp32 activations.  The inverse is built in fp32.
//
// Per-key-channel decay uses products of per-token factors exp(g) <= 1
// referenced to 16-token block boundaries, so no factor exceeds 1 except the
// inverse-prefix operand of the diagonal blocks: balanced by sqrt of the block
// factor it stays within exp(+-8) (fp16) when a block decays by at most
// exp(-16); a chunk with a steeper block uses a bf16 copy instead (fp32
// range: the decay over 16 tokens must stay above about -87 in every channel).
//
// Accumulator layout of a 16x16 MFMA result: lane l holds rows 4*(l/16)+j,
// j = 0..3, of column l%16.  The k index of an MFMA is a sum, so A and B may
// use any common permutation of it; products with a register operand use
// k = 4*(l/16)+j within each 16-wide k block, which lets an accumulator tile
// be fed back as the B operand (or, read transposed, as the A operand) of the
// next product without an LDS round trip.
#pragma once

#include "chunked_layout.h"
#include "common.h"
#include "launch.h"

namespace kda {
namespace chunked {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr float kSafeBlockDecay = 1.1253517e-07f;   // exp(-16)

// Barrier over LDS only: outstanding global loads (the next chunk's prefetch)
// stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

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
  __device__ static void mma(f32x4& acc, const frag& a, const frag& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc, 0, 0, 0);
  }
  __device__ static void scale_cont(frag& f, const float* v, int k0, int g) {
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = (T)(static_cast<float>(f[e]) * v[k0 + 8 * g + e]);
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
  __device__ static void mma(f32x4& acc, const frag& a, const frag& b) {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[j], b.lo[j], acc, 0, 0, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[j], b.hi[j], acc, 0, 0, 0);
  }
  __device__ static void scale_cont(frag& f, const float* v, int k0, int g) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f.lo[e] *= v[k0 + 4 * g + e];
      f.hi[e] *= v[k0 + 16 + 4 * g + e];
    }
  }
};

// bf16 x bf16 product for the diagonal-block Gram of a steep per-channel
// chunk.  Whole-vector bit casts: building a __bf16 vector element by element
// from 16-bit patterns is not reliably compiled.
__device__ __forceinline__ void mma_diag_bf16(f32x4& acc, const f16x8& a_f16,
                                              const uint16_t* kinv_row, int k0, int g) {
  const uint4 braw = *reinterpret_cast<const uint4*>(kinv_row + k0 + 8 * g);
  uint32_t aw[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t lo = f32_to_bf16(static_cast<float>(a_f16[2 * e]));
    const uint32_t hi = f32_to_bf16(static_cast<float>(a_f16[2 * e + 1]));
    aw[e] = lo | (hi << 16);
  }
  const uint4 araw = uint4{aw[0], aw[1], aw[2], aw[3]};
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, araw),
                                               __builtin_bit_cast(bf16x8, braw), acc, 0, 0, 0);
}

template <typename In> struct OpOf { using T = _Float16; using KinvT = uint16_t; };
template <> struct OpOf<float> { using T = float; using KinvT = float; };

struct ChunkParams {
  const void* q; const void* k; const void* v; const void* beta; const void* decay;
  const float* init; float* o; float* state;
  int T, H, DV, nsl, xcd_map, decay_kind, l2norm;
  float scale;
};

// Lower-triangular block pair (i, j), j <= i, of pair index n.
__host__ __device__ constexpr int pair_i(int n) { int i = 0; while (n > i) { n -= i + 1; ++i; } return i; }
__host__ __device__ constexpr int pair_j(int n) { int i = 0; while (n > i) { n -= i + 1; ++i; } return n; }

// ------------------------------------------------------------------ kernel --

// Transposed 4 x fp16 read (gfx950 ds_read_b64_tr_b16).  Within each group of
// 16 lanes, lane j supplies the address of an 8-byte row piece E_j; lane
// i = 4a + e receives (E_a[e], E_{a+4}[e], E_{a+8}[e], E_{a+12}[e]).
__device__ __forceinline__ f16x4 ld_tr16(const _Float16* p) {
  typedef short s4 __attribute__((ext_vector_type(4)));
  const s4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s4*)(p));
  return __builtin_bit_cast(f16x4, v);
}

// A operand of a product contracting over tokens, read from a row-major
// [tokens][channels] tile: lane (g, l16) gets channel c0 + l16 at tokens
// k0 + 4g + j and k0 + 16 + 4g + j (the "perm" k map).  Without `hi` the
// tile ends at k0 + 16 and the second half is zero.
__device__ __forceinline__ f16x8 ld_tokens(const _Float16* tile, int ld, int k0, int c0,
                                           int g, int l16, bool hi) {
  const _Float16* p = tile + (k0 + 4 * g + (l16 >> 2)) * ld + c0 + 4 * (l16 & 3);
  const f16x4 lo = ld_tr16(p);
  const f16x4 up = hi ? ld_tr16(p + 16 * ld) : f16x4{0, 0, 0, 0};
  return __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ Mma<float>::frag ld_tokens(const float* tile, int ld, int k0, int c0,
                                                      int g, int l16, bool hi) {
  Mma<float>::frag f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f.lo[j] = tile[(k0 + 4 * g + j) * ld + c0 + l16];
    f.hi[j] = hi ? tile[(k0 + 16 + 4 * g + j) * ld + c0 + l16] : 0.f;
  }
  return f;
}

template <int DK, int DVS, int C, typename In, int DECAY>
__global__ __launch_bounds__(kThreads, 1) void chunked_kernel(ChunkParams p) {
  using OpT = typename OpOf<In>::T;
  using KinvT = typename OpOf<In>::KinvT;
  using M = Mma<OpT>;
  using L = ChunkLayout<DK, DVS, C, sizeof(OpT)>;
  constexpr int NB = L::NB;
  constexpr int V = act<In>::kVec;           // activation elements per 16-byte load
  constexpr int LPR = DK / V;                // lanes per q/k row
  constexpr int RPP = kThreads / LPR;        // q/k rows per load pass
  constexpr int NP = (C + RPP - 1) / RPP;    // q/k load passes
  constexpr int LPRv = DVS / V;
  constexpr int RPPv = kThreads / LPRv;
  constexpr int NPv = (C + RPPv - 1) / RPPv;
  constexpr int NKT = DK / 16;               // 16-row tiles of the state
  constexpr int NKP = DK / 32;               // 32-wide k steps over the key dim
  constexpr int NPAIR = NB * (NB + 1) / 2;
  constexpr int NOWN = DVS / 16;             // waves that own state columns
  constexpr int NH = (NB + 1) / 2;           // 32-wide k steps over the chunk's tokens
  static_assert(LPR <= 64 && (64 % LPR) == 0, "q/k rows must pack into waves");
  static_assert(LPRv >= 1 && (64 % LPRv) == 0, "v rows must pack into waves");
  static_assert(DVS % 16 == 0 && NOWN <= kWaves, "slice width");
  // one kernel per decay kind keeps the chunk loop small enough for the
  // instruction cache
  constexpr bool chan = DECAY == DECAY_CHANNEL;
  constexpr bool headdecay = DECAY == DECAY_HEAD;

  extern __shared__ __align__(256) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int T = p.T, H = p.H, DV = p.DV;

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
  OpT* sK = reinterpret_cast<OpT*>(smem + L::oK);
  OpT* sV = reinterpret_cast<OpT*>(smem + L::oV);
  OpT* sP = reinterpret_cast<OpT*>(smem + L::oP);
  float* sAm = reinterpret_cast<float*>(smem + L::oAM);
  OpT* sGst = reinterpret_cast<OpT*>(smem + L::oAM);     // staged per-channel gate [C][DK]
  float* sTm = reinterpret_cast<float*>(smem + L::oRA);
  OpT* sTu = reinterpret_cast<OpT*>(smem + L::oTu);
  OpT* sKb = reinterpret_cast<OpT*>(smem + L::oRA);
  KinvT* sKinv = reinterpret_cast<KinvT*>(smem + L::oKinv);
  OpT* sKF = reinterpret_cast<OpT*>(smem + L::oKF(true));
  float* sv = reinterpret_cast<float*>(smem + L::oVec(chan));
  float* s_bt = sv;
  float* s_Gi = sv + C;
  float* s_Ge = sv + 2 * C;
  float* s_eG = sv + 3 * C;
  float* s_eGx = sv + 4 * C;
  float* s_eF = sv + 5 * C;
  float* s_misc = sv + 6 * C;                  // [0] = exp(G_last), [1] = steep-gate flag
  int* s_flag = reinterpret_cast<int*>(s_misc + 1);
  float* s_tau = s_misc + 16;                  // [NB][DK] whole-block decay factors
  float* s_Cb = s_tau + NB * DK;               // [NB][DK] decay of all earlier blocks
  float* s_rsq = s_Cb + NB * DK;               // [NB][DK] 1/sqrt(block factor)
  float* s_D = s_rsq + NB * DK;                // [ND][DK] decay strictly between blocks
  float* s_decC = s_D + L::ND * DK;            // [DK] decay of the whole chunk

  // Zero all of LDS once: padding columns and never-written blocks read as zero.
  {
    constexpr int nvec = static_cast<int>(L::bytes(chan) / 16);
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
  // kept as raw activation values: converting right after the load would make
  // the compiler wait for every outstanding load, the prefetch included
  In rbeta{}, rgh{};

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
    rbeta = In{}; rgh = In{};
    if (tid < C && tid < Lc) {
      const long off = (tok0 + t0 + tid) * H + h;
      rbeta = gb[off];
      if (headdecay) rgh = gg[off];
    }
  };
  auto unpack = [&](const uint4& raw, float (&x)[V]) {
    act<In>::load_vec(reinterpret_cast<const In*>(&raw), x);
  };
  auto store_row = [&](OpT* dst, const float (&x)[V]) {
    if constexpr (sizeof(OpT) == 2) {
      f16x8 hv;
#pragma unroll
      for (int e = 0; e < 8; ++e) hv[e] = (_Float16)x[e];
      *reinterpret_cast<f16x8*>(dst) = hv;
    } else {
      *reinterpret_cast<f32x4*>(dst) = f32x4{x[0], x[1], x[2], x[3]};
    }
  };

  // ---- the state slice: owner wave w keeps value columns n0 + 16w .. +15 ----
  const bool owner = wave < NOWN;
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
  lds_barrier();   // LDS zero-fill visible

  for (int ch = 0; ch < nchunks; ++ch) {
    const int t0 = ch * C;
    const int Lc = min(C, T - t0);

    // ============ phase 1: stage the chunk: normalised rows, gates ============
#pragma unroll
    for (int pp = 0; pp < NP; ++pp) {
      const int r = pp * RPP + tid / LPR, seg = tid % LPR;
      float qv[V], kv[V];
      unpack(rq[pp], qv);
      unpack(rk[pp], kv);
      float fq = p.scale, fk = 1.f;
      if (p.l2norm) {
        // row norms: the LPR lanes of a row are consecutive, reduce with DPP moves
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int e = 0; e < V; ++e) { sq += qv[e] * qv[e]; sk += kv[e] * kv[e]; }
        fq *= inv_norm(dpp_group_sum<LPR>(sq));
        fk = inv_norm(dpp_group_sum<LPR>(sk));
      }
#pragma unroll
      for (int e = 0; e < V; ++e) { qv[e] *= fq; kv[e] *= fk; }
      if (r < C) {
        store_row(sQ + r * L::LDK + seg * V, qv);
        store_row(sK + r * L::LDK + seg * V, kv);
        if (chan) {
          float gvv[V];
          unpack(rg[pp], gvv);
          store_row(sGst + r * DK + seg * V, gvv);
        }
      }
    }
#pragma unroll
    for (int pp = 0; pp < NPv; ++pp) {
      const int r = pp * RPPv + tid / LPRv, seg = tid % LPRv;
      if (r < C) {
        float vv[V];
        unpack(rv[pp], vv);
        store_row(sV + r * L::LDV + seg * V, vv);
      }
    }
    if (wave == 0) {
      // beta and the scalar gate: lane r holds token r of the chunk (C <= 64).
      float G = (lane < C) ? act<In>::cvt(rgh) : 0.f;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(G, off, 64);
        if (lane >= off) G += y;
      }
      float Gx = __shfl_up(G, 1, 64);
      if (lane == 0) Gx = 0.f;
      const float Glast = __shfl(G, 63, 64);
      if (lane < C) {
        s_bt[lane] = act<In>::cvt(rbeta);
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
    lds_barrier();

    if (chan) {
      // (1b) per (16-token block, key channel): normalised q, k times exp(g)
      // products referenced to the block start (prefix) and end (suffix);
      // all of them are <= 1.
      constexpr int NT = (NB * DK + kThreads - 1) / kThreads;
      uint32_t kin16[NT][8];   // bf16 copy of the inverse-prefix operand, two per register
#pragma unroll
      for (int it = 0; it < NT; ++it) {
        const int task = tid + it * kThreads;
        if (task < NB * DK) {
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
            // diagonal blocks pair a factor <= 1 with its inverse; balanced by
            // sqrt(block factor) both stay within exp(+-8) for a block factor
            // >= exp(-16), which fp16 holds
            const float rs = sqrtf(pre);
            s_rsq[i * DK + c] = 1.f / rs;
#pragma unroll
            for (int t = 0; t < 16; ++t)
              *reinterpret_cast<_Float16*>(&sKinv[(16 * i + t) * L::LDK + c]) = (_Float16)(kin[t] * rs);
#pragma unroll
            for (int t = 0; t < 8; ++t)
              kin16[it][t] = static_cast<uint32_t>(f32_to_bf16(kin[2 * t])) |
                             (static_cast<uint32_t>(f32_to_bf16(kin[2 * t + 1])) << 16);
            if (pre < kSafeBlockDecay) *s_flag = 1;
          } else {
#pragma unroll
            for (int t = 0; t < 16; ++t) sKinv[(16 * i + t) * L::LDK + c] = kin[t];
          }
        }
      }
      lds_barrier();
      const bool steep = *s_flag != 0;
      // (1c) chunk-level factors and k decayed to the chunk end
#pragma unroll
      for (int it = 0; it < NT; ++it) {
        const int task = tid + it * kThreads;
        if (task < NB * DK) {
          const int i = task / DK, c = task % DK;
          const float tau = s_tau[i * DK + c];
          if constexpr (sizeof(OpT) == 2) {
            if (steep) {
#pragma unroll
              for (int t = 0; t < 16; ++t)
                sKinv[(16 * i + t) * L::LDK + c] = static_cast<uint16_t>(kin16[it][t >> 1] >> (16 * (t & 1)));
            }
          }
          float cb = 1.f, ca = 1.f;
#pragma unroll
          for (int j = 0; j < NB; ++j) {
            const float tj = s_tau[j * DK + c];
            if (j < i) cb *= tj;
            if (j > i) ca *= tj;
          }
          s_Cb[i * DK + c] = cb;
          if (i == 0) s_decC[c] = ca * tau;
          float dd = 1.f;
#pragma unroll
          for (int j = NB - 1; j >= 0; --j) {    // D[i][j] = prod_{j < m < i} tau_m
            if (j < i - 1) s_D[L::dslot(i, j) * DK + c] = dd;
            if (j < i) dd *= s_tau[j * DK + c];
          }
#pragma unroll
          for (int t = 0; t < 16; ++t) {
            const int r = 16 * i + t;
            sKF[r * L::LDK + c] = (OpT)(static_cast<float>(sKb[r * L::LDK + c]) * ca);
          }
        }
      }
      lds_barrier();
    }

    // ============ phase 2: Gram A (strictly lower) and P (lower inclusive) ============
    for (int job = wave; job < 2 * NPAIR; job += kWaves) {
      const bool isP = job >= NPAIR;
      const int i = pair_i(isP ? job - NPAIR : job), j = pair_j(isP ? job - NPAIR : job);
      const OpT* arow = (isP ? sQ : sK) + (16 * i + l16) * L::LDK;
      f32x4 acc = {0, 0, 0, 0};
      if (!chan) {
        const OpT* brow = sK + (16 * j + l16) * L::LDK;
        typename M::frag fa[NKP], fb[NKP];
#pragma unroll
        for (int m = 0; m < NKP; ++m) { fa[m] = M::ld_cont(arow, 32 * m, g); fb[m] = M::ld_cont(brow, 32 * m, g); }
#pragma unroll
        for (int m = 0; m < NKP; ++m) M::mma(acc, fa[m], fb[m]);
      } else if (i == j) {
        if constexpr (sizeof(OpT) == 2) {
          const KinvT* krow = sKinv + (16 * j + l16) * L::LDK;
          if (*s_flag == 0) {
            const OpT* krh = reinterpret_cast<const OpT*>(krow);
#pragma unroll
            for (int m = 0; m < NKP; ++m) {
              auto fa = M::ld_cont(arow, 32 * m, g);
              M::scale_cont(fa, s_rsq + i * DK, 32 * m, g);
              M::mma(acc, fa, M::ld_cont(krh, 32 * m, g));
            }
          } else {
#pragma unroll
            for (int m = 0; m < NKP; ++m) mma_diag_bf16(acc, M::ld_cont(arow, 32 * m, g), krow, 32 * m, g);
          }
        } else {
          const OpT* krow = sKinv + (16 * j + l16) * L::LDK;
#pragma unroll
          for (int m = 0; m < NKP; ++m) M::mma(acc, M::ld_cont(arow, 32 * m, g), M::ld_cont(krow, 32 * m, g));
        }
      } else {
        const OpT* brow = sKb + (16 * j + l16) * L::LDK;
#pragma unroll
        for (int m = 0; m < NKP; ++m) {
          auto fa = M::ld_cont(arow, 32 * m, g);
          if (i - j >= 2) M::scale_cont(fa, s_D + L::dslot(i, j) * DK, 32 * m, g);
          M::mma(acc, fa, M::ld_cont(brow, 32 * m, g));
        }
      }
      const int s = 16 * j + l16;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int r = 16 * i + 4 * g + jj;
        if (!isP) {
          float val = acc[jj] * s_bt[r];
          if (headdecay) val *= __expf(s_Ge[r] - s_Gi[s]);
          sAm[r * L::LF + s] = (i > j || s < r) ? val : 0.f;
        } else {
          float val = acc[jj];
          if (headdecay) val *= __expf(s_Gi[r] - s_Gi[s]);
          sP[r * L::LC + s] = (OpT)((i > j || s <= r) ? val : 0.f);
        }
      }
    }
    lds_barrier();

    // ============ phase 3: T = (I + A)^-1, stored as T (fp32) and T diag(beta) ============
    if (wave == 0) {
      // diagonal 16x16 blocks, lane -> (block, column): right-looking
      // substitution, so each step leaves only independent updates behind
      const int i = g, jc = l16;
      if (i < NB) {
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = (r == jc) ? 1.f : 0.f;
        const float* ablk = sAm + (16 * i) * L::LF + 16 * i;
#pragma unroll
        for (int s = 0; s < 15; ++s) {
#pragma unroll
          for (int r = s + 1; r < 16; ++r) x[r] -= ablk[r * L::LF + s] * x[s];
        }
        const float bj = s_bt[16 * i + jc];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          sTm[(16 * i + r) * L::LF + 16 * i + jc] = x[r];
          sTu[(16 * i + r) * L::LC + 16 * i + jc] = (OpT)(x[r] * bj);
        }
      }
    } else if (chan) {
      // T diag(beta) shares its LDS with the Gram factors: zero it above the
      // block diagonal (and past the chunk for C = 16)
      for (int idx = tid - 64; idx < C * L::NCOL; idx += kThreads - 64) {
        const int r = idx / L::NCOL, s = idx % L::NCOL;
        if ((s >> 4) > (r >> 4)) sTu[r * L::LC + s] = (OpT)0.f;
      }
      {
        // chunk-referenced decays for the state step: K * exp(Gx), Q * exp(G)
        constexpr int VE = sizeof(OpT) == 2 ? 8 : 4;
        for (int idx = tid - 64; idx < C * DK / VE; idx += kThreads - 64) {
          const int r = idx / (DK / VE), c = (idx % (DK / VE)) * VE;
          const float* cb = s_Cb + (r >> 4) * DK + c;
          OpT* kp = sK + r * L::LDK + c;
          OpT* qp = sQ + r * L::LDK + c;
#pragma unroll
          for (int e = 0; e < VE; ++e) {
            kp[e] = (OpT)(static_cast<float>(kp[e]) * cb[e]);
            qp[e] = (OpT)(static_cast<float>(qp[e]) * cb[e]);
          }
        }
      }
    }
    lds_barrier();
#pragma unroll
    for (int d = 1; d < NB; ++d) {
      // blocks on diagonal d: T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj, on waves 1..
      const int j = wave - 1, i = j + d;
      if (wave >= 1 && i < NB) {
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
        const float bj = s_bt[16 * j + l16];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int r = 16 * i + 4 * g + jj;
          sTm[r * L::LF + 16 * j + l16] = -Y[jj];
          sTu[r * L::LC + 16 * j + l16] = (OpT)(-Y[jj] * bj);
        }
      }
      lds_barrier();
    }

    // ============ phase 4: state step and output (owner waves) ============
    if (owner) {
      typename M::frag Sf[NKP];
#pragma unroll
      for (int m = 0; m < NKP; ++m) Sf[m] = M::from_acc(S[2 * m], S[2 * m + 1]);
      // X = V - diag(sk exp(Gx)) K S0, one 16-token tile at a time
      f32x4 Xl[NB];
      const OpT* vcol = sV + 16 * wave + l16;
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) {
        f32x4 acc = {0, 0, 0, 0};
        const OpT* krow = sK + (16 * rt + l16) * L::LDK;
        typename M::frag fk[NKP];
#pragma unroll
        for (int m = 0; m < NKP; ++m) fk[m] = M::ld_perm(krow, 32 * m, g);
#pragma unroll
        for (int m = 0; m < NKP; ++m) M::mma(acc, fk[m], Sf[m]);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int r = 16 * rt + 4 * g + jj;
          float ks = acc[jj];
          if (headdecay) ks *= s_eGx[r];
          Xl[rt][jj] = static_cast<float>(vcol[r * L::LDV]) - ks;
        }
      }
      // D = T diag(beta) X
      typename M::frag Xf[NH];
#pragma unroll
      for (int m = 0; m < NH; ++m)
        Xf[m] = M::from_acc(Xl[2 * m], 2 * m + 1 < NB ? Xl[2 * m + 1] : f32x4{0, 0, 0, 0});
      f32x4 Dl[NB];
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) {
        Dl[rt] = f32x4{0, 0, 0, 0};
        const OpT* urow = sTu + (16 * rt + l16) * L::LC;
#pragma unroll
        for (int m = 0; m <= rt / 2; ++m) M::mma(Dl[rt], M::ld_perm(urow, 32 * m, g), Xf[m]);
      }
      typename M::frag Df[NH];
#pragma unroll
      for (int m = 0; m < NH; ++m)
        Df[m] = M::from_acc(Dl[2 * m], 2 * m + 1 < NB ? Dl[2 * m + 1] : f32x4{0, 0, 0, 0});
      // O^T = S0^T (diag(sq exp(G)) Q)^T + D^T P^T, one 16-token tile at a time
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) {
        const OpT* qrow = sQ + (16 * rt + l16) * L::LDK;
        typename M::frag fq[NKP];
#pragma unroll
        for (int m = 0; m < NKP; ++m) fq[m] = M::ld_perm(qrow, 32 * m, g);
        f32x4 acc = {0, 0, 0, 0};
#pragma unroll
        for (int m = 0; m < NKP; ++m) M::mma(acc, Sf[m], fq[m]);
        const int r = 16 * rt + l16;
        if (headdecay) acc *= s_eG[r];
        const OpT* prow = sP + r * L::LC;
#pragma unroll
        for (int m = 0; m <= rt / 2; ++m) M::mma(acc, Df[m], M::ld_perm(prow, 32 * m, g));
        if (r < Lc) {
          float* op = p.o + ((tok0 + t0 + r) * H + h) * static_cast<long>(DV) + n0 + 16 * wave + 4 * g;
          *reinterpret_cast<f32x4*>(op) = acc;
        }
      }
      // S <- exp(G_last) S0 + KY D', KY = (diag(sk exp(G_last - G)) K)^T
#pragma unroll
      for (int t = 0; t < NKT; ++t) {
        if (chan) {
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) S[t][jj] *= s_decC[16 * t + 4 * g + jj];
        } else if (headdecay) {
          S[t] *= s_misc[0];
        }
      }
      if (headdecay) {
#pragma unroll
        for (int st = 0; st < NB; ++st) {
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) Dl[st][jj] *= s_eF[16 * st + 4 * g + jj];
        }
#pragma unroll
        for (int m = 0; m < NH; ++m)
          Df[m] = M::from_acc(Dl[2 * m], 2 * m + 1 < NB ? Dl[2 * m + 1] : f32x4{0, 0, 0, 0});
      }
      const OpT* KY = chan ? sKF : sK;
#pragma unroll
      for (int t = 0; t < NKT; ++t) {
#pragma unroll
        for (int m = 0; m < NH; ++m)
          M::mma(S[t], ld_tokens(KY, L::LDK, 32 * m, 16 * t, g, l16, 2 * m + 1 < NB), Df[m]);
      }
    }
    lds_barrier();
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

template <int DK, int DVS, int C, typename In, int DECAY>
hipError_t launch_one(const ChunkParams& cp, int nwg, hipStream_t s) {
  using OpT = typename OpOf<In>::T;
  using L = ChunkLayout<DK, DVS, C, sizeof(OpT)>;
  constexpr bool chan = DECAY == DECAY_CHANNEL;
  if constexpr (L::bytes(chan) > kMaxLds) {
    return hipErrorInvalidConfiguration;   // never instantiated as a kernel
  } else {
    auto fn = chunked_kernel<DK, DVS, C, In, DECAY>;
    static bool attr_set = false;   // benign race: the attribute call is idempotent
    if (!attr_set) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                         hipFuncAttributeMaxDynamicSharedMemorySize,
                                         static_cast<int>(kMaxLds));
      if (e != hipSuccess) return e;
      attr_set = true;
    }
    fn<<<dim3(nwg), dim3(kThreads), L::bytes(chan), s>>>(cp);
    return hipGetLastError();
  }
}

template <int OpBytes>
size_t lds_bytes(int DK, int DVS, int C, bool chan) {
#define KDA_L(dk, dvs, c) \
  if (DK == dk && DVS == dvs && C == c) return ChunkLayout<dk, dvs, c, OpBytes>::bytes(chan);
#define KDA_L2(dk, c) KDA_L(dk, 16, c) KDA_L(dk, 32, c) KDA_L(dk, 64, c)
#define KDA_L3(c) KDA_L2(32, c) KDA_L2(64, c) KDA_L2(128, c)
  KDA_L3(16) KDA_L3(32) KDA_L3(64)
#undef KDA_L3
#undef KDA_L2
#undef KDA_L
  return 0;
}

template <typename In, int DECAY>
hipError_t launch_any(int DK, int DVS, int C, const ChunkParams& cp, int nwg, hipStream_t s) {
#define KDA_C(dk, dvs, c) \
  if (DK == dk && DVS == dvs && C == c) return launch_one<dk, dvs, c, In, DECAY>(cp, nwg, s);
#define KDA_C2(dk, c) KDA_C(dk, 16, c) KDA_C(dk, 32, c) KDA_C(dk, 64, c)
#define KDA_C3(c) KDA_C2(32, c) KDA_C2(64, c) KDA_C2(128, c)
  KDA_C3(16) KDA_C3(32) KDA_C3(64)
#undef KDA_C3
#undef KDA_C2
#undef KDA_C
  return hipErrorInvalidValue;
}

// One instantiation unit per (activation dtype, decay kind): chunked_<dtype>_d<kind>.hip.
#define KDA_DECLARE_LAUNCH(name) \
  hipError_t name(int DK, int DVS, int C, const ChunkParams& cp, int nwg, hipStream_t s);
KDA_DECLARE_LAUNCH(launch_bf16_d0)
KDA_DECLARE_LAUNCH(launch_bf16_d1)
KDA_DECLARE_LAUNCH(launch_bf16_d2)
KDA_DECLARE_LAUNCH(launch_f32_d0)
KDA_DECLARE_LAUNCH(launch_f32_d1)
KDA_DECLARE_LAUNCH(launch_f32_d2)
#undef KDA_DECLARE_LAUNCH

}  // namespace chunked
}  // namespace kda
