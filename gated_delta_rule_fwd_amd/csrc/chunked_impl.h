// Chunked forward of the gated delta rule on gfx950 (kernel templates).
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
// Two kernels on the caller's stream:
//
//  * prep_kernel, one workgroup per (sequence, head, chunk), all chunks in
//    parallel: normalisation, gate cumsums, A and P on MFMA, the inverse, and
//    the decayed operands.  It writes one record per chunk to a workspace:
//    Q, K (and for per-channel decay K * exp(G_last - G)), T diag(beta), P and
//    the per-token / per-channel decay factors.
//  * state_kernel, one workgroup per (sequence, head, slice of DVS value
//    columns), walks the chunks in order.  Its DVS/16 "owner" waves keep 16
//    columns of S each in MFMA accumulators for the whole sequence; per chunk
//    the workgroup stages the record into LDS (prefetched into registers one
//    chunk ahead) and the owner waves form D, the output rows and the new state.
//
// MFMA: v_mfma_f32_16x16x32_f16 for bf16 activations (q, k normalised and v
// rounded once to fp16; derived operands rounded once to fp16) and
// v_mfma_f32_16x16x4_f32 for fp32 activations.  The inverse is built in fp32.
//
// Per-key-channel decay.  A chunk whose every 4-token quarter decays by at
// most e^-3 in every channel (mild decay) takes each 16-token block's
// operands referenced to its middle token, within e^6 of the row, and one
// product per block pair.  Any other chunk takes the exact path, which uses
// products of per-token factors exp(g) <= 1 only,
// so no operand exceeds the normalised row it scales, whatever the decay
// (exp(g) may underflow to 0: the products it belongs to are then 0, as
// they should be to well below fp16 resolution).  A Gram entry of tokens
// s < r carries the decay of the tokens strictly between them (A) or of
// s+1 .. r (P).  Between 16-token blocks it is split as (k_s decayed to the
// end of its block) x (the decay of the blocks in between, an fp32 scale) x
// (the row decayed from the start of its block).  Within a diagonal block
// the same split is made at 4-token quarters (one MFMA pass per column
// quarter), and the pairs inside one quarter are summed over the channels
// directly in fp32.
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

#include <utility>

namespace kda {
namespace chunked {

constexpr int kThreads = 256;
constexpr int kWaves = 4;

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
  // times v1 (if u1) and v2 (if u2) per k, rounded once
  __device__ static void scale_cont2(frag& f, const float* v1, bool u1, const float* v2, bool u2, int k0,
                                     int g) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float a = u1 ? v1[k0 + 8 * g + e] : 1.f, b = u2 ? v2[k0 + 8 * g + e] : 1.f;
      f[e] = (T)(static_cast<float>(f[e]) * (a * b));
    }
  }
  __device__ static frag zero() { return frag{0, 0, 0, 0, 0, 0, 0, 0}; }
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
  __device__ static void scale_cont2(frag& f, const float* v1, bool u1, const float* v2, bool u2, int k0,
                                     int g) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a0 = u1 ? v1[k0 + 4 * g + e] : 1.f, b0 = u2 ? v2[k0 + 4 * g + e] : 1.f;
      const float a1 = u1 ? v1[k0 + 16 + 4 * g + e] : 1.f, b1 = u2 ? v2[k0 + 16 + 4 * g + e] : 1.f;
      f.lo[e] *= a0 * b0;
      f.hi[e] *= a1 * b1;
    }
  }
  __device__ static frag zero() { return frag{f32x4{0, 0, 0, 0}, f32x4{0, 0, 0, 0}}; }
};

// bf16 operand of 8 elements from two accumulator tiles (rows 4g..4g+3 of
// each), rounded to nearest even; and the bf16 product.
__device__ __forceinline__ bf16x8 bf_from_acc(const f32x4& a, const f32x4& b) {
  return bf16x8{(__bf16)a[0], (__bf16)a[1], (__bf16)a[2], (__bf16)a[3],
                (__bf16)b[0], (__bf16)b[1], (__bf16)b[2], (__bf16)b[3]};
}
// The rounding remainder of bf_from_acc(a, b) == hi, itself rounded to bf16:
// hi + lo carries about 16 significant bits.
__device__ __forceinline__ bf16x8 bf_lo(const f32x4& a, const f32x4& b, const bf16x8& hi) {
  return bf16x8{(__bf16)(a[0] - (float)hi[0]), (__bf16)(a[1] - (float)hi[1]),
                (__bf16)(a[2] - (float)hi[2]), (__bf16)(a[3] - (float)hi[3]),
                (__bf16)(b[0] - (float)hi[4]), (__bf16)(b[1] - (float)hi[5]),
                (__bf16)(b[2] - (float)hi[6]), (__bf16)(b[3] - (float)hi[7])};
}
__device__ __forceinline__ void mma_bf(f32x4& acc, const bf16x8& a, const bf16x8& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}
// acc + the sum of squares of the 8 elements of x (fp32, in pairs)
__device__ __forceinline__ float sumsq_bf(const bf16x8& x, float acc) {
  const bf16x2 a = __builtin_shufflevector(x, x, 0, 1), b = __builtin_shufflevector(x, x, 2, 3);
  const bf16x2 c = __builtin_shufflevector(x, x, 4, 5), d = __builtin_shufflevector(x, x, 6, 7);
  acc = __builtin_amdgcn_fdot2_f32_bf16(a, a, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(b, b, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(c, c, acc, false);
  return __builtin_amdgcn_fdot2_f32_bf16(d, d, acc, false);
}
template <typename In> struct OpOf { using T = _Float16; };
template <> struct OpOf<float> { using T = float; };

// Packed variable-length input (B = 1, N sequences back to back in T): cu
// holds the N + 1 token offsets of the sequences, cb the N + 1 offsets of
// their chunks (chunks never cross a sequence end); nchunks is then the total
// chunk count.  NULL cu: N = B sequences of T tokens each.
struct PrepParams {
  const void* q; const void* k; const void* beta; const void* decay;
  unsigned char* ws;     // records, [B*H][nchunks] ([H][chunks] packed)
  int T, H, nchunks, l2norm;
  int c0;                // first chunk of this launch (records are indexed from it)
  float scale;
  const int* cu; const int* cb; int nseq;   // packed input
  Transforms tf;         // raw gate / raw beta (applied where decay and beta are read)
  int Hk;                // q/k heads: value head h reads q, k head h / (H / Hk)
  unsigned long long hk_magic;   // ceil(2^32 / (H / Hk)): that head is (h * hk_magic) >> 32
};

// q/k head of value head h, (h * ceil(2^32 / g)) >> 32 = h / g exactly for
// h, g < 2^16 (the error term h * e / 2^32, e < g, stays below 1 / g)
__device__ __forceinline__ int qk_head(int h, unsigned long long magic) {
  return static_cast<int>((static_cast<unsigned long long>(h) * magic) >> 32);
}

struct StateParams {
  const void* q; const void* k;   // raw q, k rows (records without Q, K tiles)
  const void* v; const unsigned char* ws;
  const float* init; float* o; float* state;
  int T, H, DV, nchunks, nsl, xcd_map;
  int c0;                // first chunk of this launch; `init` holds the state entering it
  int l2norm; float scale;   // q's row factor (raw rows)
  const int* cu; const int* cb;   // packed input (see PrepParams); state and o by sequence
  int Hk;                // q/k heads (see PrepParams)
  unsigned long long hk_magic;
  int vfirst;            // init and state value-major [.., H, DV, DK]
};

// The sequence of packed chunk g: the last n with cb[n] <= g (cb
// nondecreasing, cb[0] = 0 <= g < cb[nseq]).
__device__ __forceinline__ int seq_of_chunk(const int* cb, int nseq, int g) {
  int lo = 0, hi = nseq;   // cb[lo] <= g < cb[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cb[mid] <= g) lo = mid;
    else hi = mid;
  }
  return lo;
}

// Lower-triangular block pair (i, j), j <= i, of pair index n.
__host__ __device__ constexpr int pair_i(int n) { int i = 0; while (n > i) { n -= i + 1; ++i; } return i; }
__host__ __device__ constexpr int pair_j(int n) { int i = 0; while (n > i) { n -= i + 1; ++i; } return n; }
// f(std::integral_constant<int, i>) for i = 0 .. N-1: a loop whose index is
// a compile-time constant in the body.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}
// P operand fragments of the state kernel: fragment pf_n(ib, m) holds row
// block ib at the 32-token k step m (m <= ib / 2), fragments running over ib,
// then m.  P's 16 x 16 blocks (ib, jb <= ib) in the order the helper waves
// share them: ib from the last row block down, then jb up.
__host__ __device__ constexpr int pf_n(int ib, int m) { return ib / 2 * (ib / 2 + 1) + (ib & 1) * (ib / 2 + 1) + m; }
__host__ __device__ constexpr int blk_ib(int b, int nb) { int i = nb - 1; while (b > i) { b -= i + 1; --i; } return i; }
__host__ __device__ constexpr int blk_jb(int b, int nb) { int i = nb - 1; while (b > i) { b -= i + 1; --i; } return b; }

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

// 16 bytes of operands (8 fp16 or 4 fp32) from fp32 values.
template <typename OpT, int N>
__device__ __forceinline__ void store16(OpT* dst, const float (&x)[N]) {
  if constexpr (sizeof(OpT) == 2) {
    static_assert(N == 8, "8 fp16 per 16 bytes");
    f16x8 hv;
#pragma unroll
    for (int e = 0; e < 8; ++e) hv[e] = (_Float16)x[e];
    *reinterpret_cast<f16x8*>(dst) = hv;
  } else {
    static_assert(N == 4, "4 fp32 per 16 bytes");
    *reinterpret_cast<f32x4*>(dst) = f32x4{x[0], x[1], x[2], x[3]};
  }
}

// N consecutive elements e0.. of row r of a record tile (N, e0 multiples of 4),
// placed in perm_pos order, 4 elements per store.
template <typename OpT, int PPR, int N>
__device__ __forceinline__ void put_perm(unsigned char* tile, int r, int e0, const float (&x)[N]) {
#pragma unroll
  for (int a = 0; a < N / 4; ++a) {
    unsigned char* dst = tile + swz_off<PPR>(r, perm_pos(e0 + 4 * a) * static_cast<int>(sizeof(OpT)));
    if constexpr (sizeof(OpT) == 2) {
      *reinterpret_cast<f16x4*>(dst) = f16x4{(_Float16)x[4 * a], (_Float16)x[4 * a + 1],
                                             (_Float16)x[4 * a + 2], (_Float16)x[4 * a + 3]};
    } else {
      *reinterpret_cast<f32x4*>(dst) = f32x4{x[4 * a], x[4 * a + 1], x[4 * a + 2], x[4 * a + 3]};
    }
  }
}

// ------------------------------------------------------------- prep kernel --

// Eight waves per workgroup: the chunk's work is short, so more waves hide
// the LDS and HBM latencies of its dependent phases.
constexpr int kPrepThreads = 512;
// Per-channel decay: the mild path's bound on a 4-token quarter's log decay
constexpr float kMildQuarterLog = 3.f;
constexpr int kPrepWaves = kPrepThreads / 64;

// Waves per SIMD of the prep kernel: two 8-wave workgroups share a CU with
// per-channel decay, four with raw rows (the smaller LDS plan), else three.
template <int DK, int C, typename In, int DECAY>
constexpr int prep_waves() {
  return DECAY == DECAY_CHANNEL ? 4
       : RecLayout<DK, C, sizeof(typename OpOf<In>::T), false>::kRawK ? 8 : 6;
}

// TF: the raw-gate / raw-beta transforms may be on (a separate instantiation,
// so the plain inputs pay nothing for them)
template <int DK, int C, typename In, int DECAY, bool TF>
__global__ __launch_bounds__(kPrepThreads, (prep_waves<DK, C, In, DECAY>())) void prep_kernel(PrepParams p) {
  using OpT = typename OpOf<In>::T;
  using M = Mma<OpT>;
  constexpr bool chan = DECAY == DECAY_CHANNEL;
  constexpr bool headdecay = DECAY == DECAY_HEAD;
  using R = RecLayout<DK, C, sizeof(OpT), chan>;
  using L = PrepLayout<DK, C, sizeof(OpT), R::kRawK>;
  constexpr int NB = L::NB;
  constexpr int V = act<In>::kVec;           // activation elements per 16-byte load
  static_assert(V * sizeof(OpT) == 16, "one 16-byte load makes one 16-byte operand store");
  constexpr int LPR = DK / V;                // lanes per q/k row
  constexpr int RPP = kPrepThreads / LPR;        // q/k rows per load pass
  constexpr int NP = (C + RPP - 1) / RPP;    // q/k load passes
  constexpr int NKP = DK / 32;               // 32-wide k steps over the key dim
  constexpr int NPAIR = NB * (NB + 1) / 2;
  static_assert(LPR <= 64 && (64 % LPR) == 0, "q/k rows must pack into waves");

  extern __shared__ __align__(256) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int T = p.T, H = p.H;
  const int ch = blockIdx.x % p.nchunks, head = blockIdx.x / p.nchunks;
  const int b = head / H, h = head % H;
  const int hk = qk_head(h, p.hk_magic);   // the q/k head of value head h
  int Lc;                 // tokens in the chunk
  long tok0;              // first token of the chunk
  if (p.cu) {
    const int n = seq_of_chunk(p.cb, p.nseq, ch);
    const int t0 = p.cu[n] + (ch - p.cb[n]) * C;
    Lc = min(C, p.cu[n + 1] - t0);
    tok0 = t0;
  } else {
    const int t0 = (p.c0 + ch) * C;
    Lc = min(C, T - t0);
    tok0 = static_cast<long>(b) * T + t0;
  }
  // the chunk's record image; the workspace holds its bytes from R::gOff on
  unsigned char* rec = reinterpret_cast<unsigned char*>(
      reinterpret_cast<uintptr_t>(p.ws) + (static_cast<size_t>(head) * p.nchunks + ch) * R::gBytes - R::gOff);
  float* rvec = reinterpret_cast<float*>(rec + R::oVec);

  OpT* sQ = reinterpret_cast<OpT*>(smem + L::oQ);
  OpT* sK = reinterpret_cast<OpT*>(smem + L::oK);
  float* sAm = reinterpret_cast<float*>(smem + L::oAM);
  OpT* sGst = reinterpret_cast<OpT*>(smem + L::oAM);     // staged per-channel gate [C][DK]
  float* sTm = reinterpret_cast<float*>(smem + L::oRA(chan));
  OpT* sKB = reinterpret_cast<OpT*>(smem + L::oKB);       // per-channel: k decayed to its quarter's / block's end
  float* sv = reinterpret_cast<float*>(smem + L::oVec(chan));
  float* s_bt = sv;
  float* s_Gi = sv + C;
  float* s_Ge = sv + 2 * C;
  float* s_qk = sv + 3 * C;                    // per-channel decay: q_hat . k_hat per token;
  float* s_fk = s_qk;                          // raw K: the row factor of k
  float* s_misc = sv + 4 * C;
  int* s_steep = reinterpret_cast<int*>(s_misc);   // per-channel decay: a quarter decays by more than e^-3
  int* s_dflag = reinterpret_cast<int*>(s_misc + 4);   // otherwise: [4] diagonal block i of A written
  float* s_tau4 = s_misc + 16;                 // [NQ][DK] decay factor of each 4-token quarter
                                               // (first its log, the quarter's gate sum; on the
                                               // mild path then the log decay from the chunk
                                               // start to the quarter's start)
  float* s_wq = s_tau4 + L::NQ * DK;           // [NQ][12] within-quarter Gram sums (A, then P)
  float* s_D = s_wq;                           // [NDD][DK] decay between blocks i, j (i - j >= 2), later
  float* s_tot = s_wq;                         // mild decay: [DK] the chunk's log decay

  const In* gq = static_cast<const In*>(p.q);
  const In* gk = static_cast<const In*>(p.k);
  const In* gb = static_cast<const In*>(p.beta);
  const In* gg = static_cast<const In*>(p.decay);

  // ============ phase 1: normalised q, k rows; gates ============
  {
    uint4 rq[NP], rk[NP], rg[NP];
    // raw per-channel gate: this thread's V channels of dt_bias (a thread
    // keeps its channel segment tid % LPR in every pass), loaded once
    float gbias[chan && TF ? V : 1];
    if constexpr (chan && TF) {
#pragma unroll
      for (int e = 0; e < V; ++e)
        gbias[e] = (p.tf.A_log && p.tf.dt_bias) ? p.tf.dt_bias[h * DK + (tid % LPR) * V + e] : 0.f;
    }
#pragma unroll
    for (int pp = 0; pp < NP; ++pp) {
      const int r = pp * RPP + tid / LPR, seg = tid % LPR;
      rq[pp] = rk[pp] = rg[pp] = uint4{0, 0, 0, 0};
      if (r < Lc) {
        const long off = ((tok0 + r) * H + h) * DK + seg * V;            // per value head
        const long offk = ((tok0 + r) * p.Hk + hk) * DK + seg * V;       // per q/k head
        if constexpr (!R::kRawK) rq[pp] = *reinterpret_cast<const uint4*>(gq + offk);
        rk[pp] = *reinterpret_cast<const uint4*>(gk + offk);
        if (chan) rg[pp] = *reinterpret_cast<const uint4*>(gg + off);
      }
    }
    // raw gate: -exp(A_log) of the head; tokens past the sequence end keep a
    // zero decay (the chunk-end sums run over all C rows)
    const float negA = (TF && p.tf.A_log) ? -__expf(p.tf.A_log[h]) : 0.f;
    float bt = 0.f, G = 0.f;
    if (wave == 0 && lane < Lc) {
      const long off = (tok0 + lane) * H + h;
      bt = act<In>::load1(gb + off);
      if (headdecay) G = act<In>::load1(gg + off);
      if constexpr (TF) {
        bt = beta_transform(bt, p.tf.beta_mode);
        if (headdecay && p.tf.A_log)
          G = gate_decay(G, negA, p.tf.dt_bias ? p.tf.dt_bias[h] : 0.f, p.tf.lower);
      }
    }
#pragma unroll
    for (int pp = 0; pp < NP; ++pp) {
      const int r = pp * RPP + tid / LPR, seg = tid % LPR;
      float qv[V], kv[V];
      act<In>::load_vec(reinterpret_cast<const In*>(&rq[pp]), qv);
      act<In>::load_vec(reinterpret_cast<const In*>(&rk[pp]), kv);
      float fq = p.scale, fk = 1.f;
      if (p.l2norm) {
        // row norms: the LPR lanes of a row are consecutive, reduce with DPP moves
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int e = 0; e < V; ++e) { sq += qv[e] * qv[e]; sk += kv[e] * kv[e]; }
        if constexpr (!R::kRawK) fq *= inv_norm(dpp_group_sum<LPR>(sq));
        fk = inv_norm(dpp_group_sum<LPR>(sk));
      }
#pragma unroll
      for (int e = 0; e < V; ++e) { qv[e] *= fq; kv[e] *= fk; }
      if constexpr (chan) {
        // the diagonal of P takes no decay: kept exact rather than through
        // the decay-referenced operands
        float qk = 0.f;
#pragma unroll
        for (int e = 0; e < V; ++e) qk += qv[e] * kv[e];
        qk = dpp_group_sum<LPR>(qk);
        if (r < C && seg == 0) s_qk[r] = qk;
      }
      if (r < C) {
        if constexpr (!R::kRawK) store16<OpT>(sQ + r * L::LDK + seg * V, qv);
        store16<OpT>(sK + r * L::LDK + seg * V, kv);
        if constexpr (R::kRawK) {
          // the state kernel takes q and k as they are; k's row factor goes
          // into the record's per-token vectors below (zero past the
          // sequence end, where the state kernel's rows are copies)
          if (seg == 0) s_fk[r] = r < Lc ? fk : 0.f;
        } else if (!chan) {   // final record operands already
          put_perm<OpT, R::PPRK>(rec + R::oQ, r, seg * V, qv);
          put_perm<OpT, R::PPRK>(rec + R::oK, r, seg * V, kv);
        } else {
          float gv[V];
          act<In>::load_vec(reinterpret_cast<const In*>(&rg[pp]), gv);
          if constexpr (TF) {
            if (p.tf.A_log && r < Lc) {
#pragma unroll
              for (int e = 0; e < V; ++e) gv[e] = gate_decay(gv[e], negA, gbias[e], p.tf.lower);
            }
          }
          store16<OpT>(sGst + r * DK + seg * V, gv);
        }
      }
    }
    if (chan && tid == 0) *s_steep = 0;
    if (!chan && tid < 4) s_dflag[tid] = 0;
    if (wave == 0) {
      // the scalar gate: lane r holds token r of the chunk (C <= 64); its
      // cumulative sums (zero without a per-head decay)
      float Gx = 0.f, Glast = 0.f;
      if constexpr (headdecay) {
        const WaveScan ws = wave_scan(G);
        G = ws.incl;
        Gx = ws.excl;
        Glast = ws.total;
      }
      if (lane < C) {
        s_bt[lane] = bt;
        s_Gi[lane] = G;
        s_Ge[lane] = Gx;
        if (headdecay && !R::kRawK) {
          rvec[R::vEG + lane] = __expf(G);
          rvec[R::vEGx + lane] = __expf(Gx);
          rvec[R::vEF + lane] = __expf(Glast - G);
        }
      }
      if (lane == 0 && headdecay) rvec[R::vMisc] = __expf(Glast);
    }
  }
  lds_barrier();

  if constexpr (R::kRawK) {
    // per-token record vectors, k's row factor folded into the two that
    // multiply its products
    if (wave == 0 && lane < C) {
      const float Gi = s_Gi[lane], Gl = s_Gi[C - 1];
      rvec[R::vEG + lane] = __expf(Gi);
      rvec[R::vEGx + lane] = __expf(s_Ge[lane]) * s_fk[lane];
      rvec[R::vEF + lane] = __expf(Gl - Gi) * s_fk[lane];
      rvec[R::vG + lane] = Gi;
      rvec[R::vFK + lane] = s_fk[lane];
    }
  }

  // The Gram tiles leave the MFMA transposed (row block j's rows times block
  // i's): a lane holds row r = 16 i + l16 at the four consecutive columns
  // s0 = 16 j + 4 g .. s0 + 3.  A gets beta_r and goes to LDS (strictly
  // lower); P (lower, inclusive) goes straight to the record, the state
  // kernel being its only reader.  wq: per-channel decay, the within-quarter
  // sums of a diagonal block (s and r in one quarter), added here.
  bool mild = false;   // per-channel decay on the mild path: no within-quarter sums

  // Diagonal 16x16 block i of T, column jc (this lane's): forward substitution
  // by rows, x_r = [r == jc] - sum_{s < r} A_rs x_s, A's row read four entries
  // at a time (one 16-byte read for the 16 lanes of a block), the sum in four
  // partial sums.  Row r + 1 is read while row r is summed: the scheduling
  // fence keeps those reads ahead of the sums, which would otherwise wait out
  // each row's read latency in turn.
  auto diag_inverse = [&](int i, int jc, float (&x)[16]) {
    const float* ablk = sAm + (16 * i) * L::LF + 16 * i;
    x[0] = jc == 0 ? 1.f : 0.f;
    f32x4 cur[4], nxt[4];
    cur[0] = *reinterpret_cast<const f32x4*>(ablk + L::LF);
#pragma unroll
    for (int r = 1; r < 16; ++r) {
      if (r < 15) {
#pragma unroll
        for (int s4 = 0; s4 < (r + 4) / 4; ++s4)
          nxt[s4] = *reinterpret_cast<const f32x4*>(ablk + (r + 1) * L::LF + 4 * s4);
      }
      __builtin_amdgcn_sched_barrier(0);
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s4 = 0; s4 < (r + 3) / 4; ++s4) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (4 * s4 + e < r) acc[e] += cur[s4][e] * x[4 * s4 + e];
      }
      x[r] = (r == jc ? 1.f : 0.f) - ((acc[0] + acc[1]) + (acc[2] + acc[3]));
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) cur[s4] = nxt[s4];
    }
  };
  float xd[16];   // without per-channel decay: wave 0's column of a diagonal block of T

  auto emit = [&](int i, int j, bool isP, const f32x4& acc) {
    const int r = 16 * i + l16, s0 = 16 * j + 4 * g;
    const f32x4 gs = *reinterpret_cast<const f32x4*>(s_Gi + s0);
    // same quarter (diagonal blocks of per-channel decay): local rows rl, jj
    const bool sameq = chan && !mild && i == j && (l16 >> 2) == g;
    const int rl = l16 & 3;
    const float* wq = s_wq + (4 * i + g) * L::kWQ + (isP ? 6 : 0) + rl * (rl - 1) / 2;
    if (!isP) {
      const float bt = s_bt[r], ge = s_Ge[r];
      f32x4 v;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        float val = acc[jj];
        if (sameq && jj < rl) val += wq[jj];
        val *= bt;
        if (headdecay) val *= __expf(ge - gs[jj]);
        v[jj] = (i > j || s0 + jj < r) ? val : 0.f;
      }
      *reinterpret_cast<f32x4*>(sAm + r * L::LF + s0) = v;
    } else {
      const float gi = s_Gi[r];
      float v[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        float val = acc[jj];
        if (sameq && jj < rl) val += wq[jj];
        if (headdecay) val *= __expf(gi - gs[jj]);
        if (chan && s0 + jj == r) val = s_qk[r];   // no decay on the diagonal: exact
        v[jj] = (i > j || s0 + jj <= r) ? val : 0.f;
      }
      unsigned char* dst = rec + R::oP + swz_off<R::PPRC>(r, perm_pos(s0) * static_cast<int>(sizeof(OpT)));
      if constexpr (sizeof(OpT) == 2) {
        *reinterpret_cast<f16x4*>(dst) = f16x4{(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
      } else {
        *reinterpret_cast<f32x4*>(dst) = f32x4{v[0], v[1], v[2], v[3]};
      }
    }
  };

  if constexpr (!chan) {
    // ============ phase 2: Gram A (strictly lower) and P (lower inclusive) ============
    // (raw rows: A only; the state kernel forms P).  Wave i < NB forms A's
    // diagonal block i and flags it; wave 0 inverts all of them (lane ->
    // block, column) as soon as they are flagged, while waves 1 .. 7 form
    // the remaining blocks: the inverse overlaps the rest of the Gram.
    auto gram = [&](int i, int j, bool isP) {
      const OpT* arow = (isP ? sQ : sK) + (16 * i + l16) * L::LDK;
      const OpT* brow = sK + (16 * j + l16) * L::LDK;
      f32x4 acc = {0, 0, 0, 0};
      typename M::frag fa[NKP], fb[NKP];
#pragma unroll
      for (int m = 0; m < NKP; ++m) { fa[m] = M::ld_cont(arow, 32 * m, g); fb[m] = M::ld_cont(brow, 32 * m, g); }
#pragma unroll
      for (int m = 0; m < NKP; ++m) M::mma(acc, fb[m], fa[m]);
      emit(i, j, isP, acc);
    };
    static_assert(NB < kPrepWaves, "a wave per diagonal block, and more for the rest");
    if (wave < NB) {
      gram(wave, wave, false);
      if (wave > 0) {
        // (the release orders this wave's writes of the block before the flag)
        if (lane == 0) __hip_atomic_store(&s_dflag[wave], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
      } else {
        // (waves 1 .. NB-1 are resident in the same workgroup and reach their
        // flag with no wait of their own, so this wait ends)
        for (int w = 1; w < NB; ++w)
          while (__hip_atomic_load(&s_dflag[w], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) == 0)
            __builtin_amdgcn_s_sleep(1);
        if (g < NB) diag_inverse(g, l16, xd);
      }
    }
    // the rest: A's off-diagonal blocks, then (unless raw rows) every block of
    // P, on waves 1 .. 7, those past NB first
    constexpr int NOFFB = NB * (NB - 1) / 2;
    constexpr int NREST = NOFFB + (R::kRawK ? 0 : NPAIR);
    constexpr int NRW = kPrepWaves - 1;
    const int rw = wave == 0 ? -1 : (wave - NB + NRW) % NRW;
    for (int q = rw; rw >= 0 && q < NREST; q += NRW) {
      if (q < NOFFB) gram(pair_i(q) + 1, pair_j(q), false);
      else gram(pair_i(q - NOFFB), pair_j(q - NOFFB), true);
    }
  } else {
    // Per-key-channel decay.  Quarter Q holds tokens 4Q .. 4Q+3; LPQ lanes
    // share a quarter, CPT consecutive channels each.
    constexpr int NQ = L::NQ;
    constexpr int LPQ = (kPrepThreads / NQ < DK ? kPrepThreads / NQ : DK) < 64
                            ? (kPrepThreads / NQ < DK ? kPrepThreads / NQ : DK) : 64;
    constexpr int CPT = DK / LPQ;
    static_assert(LPQ >= 4 && CPT * LPQ == DK && NQ * LPQ <= kPrepThreads, "quarter lanes");
    const int Q = tid / LPQ, c0 = (tid % LPQ) * CPT;
    const bool qt = tid < NQ * LPQ;   // this thread has a (quarter, channel group)
    // this thread's CPT channels of one row, as one LDS access
    typedef OpT opv __attribute__((ext_vector_type(CPT)));
    typedef float f32v __attribute__((ext_vector_type(CPT)));

    // (1a) per quarter and channel: the gate's running sum over the quarter
    // (kept in registers) and the quarter's sum (to LDS).  A quarter whose
    // decay exceeds e^-3 in any channel sends the chunk down the exact path.
    f32v lp[4];
    if (qt) {
      f32v run = 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const opv gv = *reinterpret_cast<const opv*>(sGst + (4 * Q + t) * DK + c0);
#pragma unroll
        for (int e = 0; e < CPT; ++e) run[e] += static_cast<float>(gv[e]);
        lp[t] = run;
      }
      *reinterpret_cast<f32v*>(s_tau4 + Q * DK + c0) = run;
      bool steep = false;
#pragma unroll
      for (int e = 0; e < CPT; ++e) steep |= !(run[e] >= -kMildQuarterLog);
      if (steep) *s_steep = 1;
    }
    lds_barrier();
    // the mild path's operands reach e^6 times a row: within fp16 for unit
    // rows and a q factor up to 4
    mild = *s_steep == 0 && (sizeof(OpT) == 4 || (p.l2norm && p.scale <= 4.f));

    if (mild) {
      // the log decay from the chunk start to every quarter start, in place,
      // and over the chunk: one thread per channel
      if (tid < DK) {
        float acc = 0.f;
#pragma unroll
        for (int q2 = 0; q2 < NQ; ++q2) {
          const float sq = s_tau4[q2 * DK + tid];
          s_tau4[q2 * DK + tid] = acc;
          acc += sq;
        }
        s_tot[tid] = acc;
      }
      lds_barrier();
      // Mild decay (every quarter's decay at least e^-3 in every channel, so
      // every half block's at least e^-6): the operands of a 16-token block b
      // are referenced to its middle, M_b = G at token 16 b + 7, so that one
      // product per block pair gives A and P.  Rows k exp(Gx - M_b) and
      // q exp(G - M_b) replace k and q, columns k exp(M_b - G) go to KB; all
      // lie within e^6 of the row.  Between blocks i > j the rows take the
      // fp32 scale exp(M_i - M_j) <= 1.
      if (qt) {
        const int blk = Q >> 2;
        // G at the quarter's start, M_b and G_last
        const f32v gq = *reinterpret_cast<const f32v*>(s_tau4 + Q * DK + c0);
        const f32v mb = *reinterpret_cast<const f32v*>(s_tau4 + (4 * blk + 2) * DK + c0);
        const f32v tot = *reinterpret_cast<const f32v*>(s_tot + c0);
        f32v emb, ef;
#pragma unroll
        for (int e = 0; e < CPT; ++e) {
          emb[e] = __expf(mb[e]);            // the record's chunk reference: exp(M_b)
          ef[e] = __expf(tot[e] - mb[e]);    // exp(G_last - M_b)
        }
        if (Q == 0) {
          f32v all;
#pragma unroll
          for (int e = 0; e < CPT; ++e) all[e] = __expf(tot[e]);
          *reinterpret_cast<f32v*>(rvec + R::vDecC + c0) = all;
        }
        // exp(Gx - M_b) of the quarter's first token; each later token's is
        // the exp(G - M_b) of the token before (the same sum, so the same value)
        f32v fkn;
#pragma unroll
        for (int e = 0; e < CPT; ++e) fkn[e] = __expf(gq[e] - mb[e]);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int r = 4 * Q + t;
          const opv kv = *reinterpret_cast<const opv*>(sK + r * L::LDK + c0);
          const opv qv = *reinterpret_cast<const opv*>(sQ + r * L::LDK + c0);
          opv rk, rq, rb;
          float xk[CPT], xq[CPT], xf[CPT];
#pragma unroll
          for (int e = 0; e < CPT; ++e) {
            const float gr = gq[e] + lp[t][e];   // G of token r
            const float fk = fkn[e], fq = __expf(gr - mb[e]), fb = __expf(mb[e] - gr);
            fkn[e] = fq;
            const float k1 = static_cast<float>(kv[e]), q1 = static_cast<float>(qv[e]);
            rk[e] = (OpT)(k1 * fk);
            rq[e] = (OpT)(q1 * fq);
            rb[e] = (OpT)(k1 * fb);
            xk[e] = k1 * fk * emb[e];
            xq[e] = q1 * fq * emb[e];
            xf[e] = k1 * fb * ef[e];
          }
          *reinterpret_cast<opv*>(sK + r * L::LDK + c0) = rk;
          *reinterpret_cast<opv*>(sQ + r * L::LDK + c0) = rq;
          *reinterpret_cast<opv*>(sKB + r * L::LDK + c0) = rb;
          if constexpr (CPT % 4 == 0) {
            put_perm<OpT, R::PPRK>(rec + R::oK, r, c0, xk);
            put_perm<OpT, R::PPRK>(rec + R::oQ, r, c0, xq);
            put_perm<OpT, R::PPRK>(rec + R::oF, r, c0, xf);
          } else {
#pragma unroll
            for (int e = 0; e < CPT; ++e) {
              const int off = swz_off<R::PPRK>(r, perm_pos(c0 + e) * static_cast<int>(sizeof(OpT)));
              *reinterpret_cast<OpT*>(rec + R::oK + off) = (OpT)xk[e];
              *reinterpret_cast<OpT*>(rec + R::oQ + off) = (OpT)xq[e];
              *reinterpret_cast<OpT*>(rec + R::oF + off) = (OpT)xf[e];
            }
          }
        }
      }
      lds_barrier();
      // the scale exp(M_i - M_j) <= 1 of each pair i > j, per channel, once
      // per workgroup: into rows of the quarter table that the operands have
      // finished with (none of the rows 4 b + 2 that hold M_b)
      constexpr int NOFF = NB * (NB - 1) / 2;
      auto fac_row = [](int pr) { return 4 * (pr / 3) + (pr % 3 == 2 ? 3 : pr % 3); };
      static_assert(NOFF <= 6 && NOFF <= L::NQ, "pair scales fit the quarter table");
      if (NOFF > 0 && tid < DK) {
        float f[NOFF > 0 ? NOFF : 1];
#pragma unroll
        for (int pr = 0; pr < NOFF; ++pr)
          f[pr] = __expf(s_tau4[(4 * (pair_i(pr) + 1) + 2) * DK + tid] - s_tau4[(4 * pair_j(pr) + 2) * DK + tid]);
#pragma unroll
        for (int pr = 0; pr < NOFF; ++pr) s_tau4[fac_row(pr) * DK + tid] = f[pr];
      }
      lds_barrier();
      // every block pair i >= j, A then P on the diagonal, then below it
      for (int job = wave; job < 2 * NB + 2 * NOFF; job += kPrepWaves) {
        bool isP;
        int i, j, pr = 0;
        if (job < 2 * NB) {
          isP = job >= NB;
          i = j = isP ? job - NB : job;
        } else {
          const int o = job - 2 * NB;
          isP = o >= NOFF;
          pr = isP ? o - NOFF : o;
          i = pair_i(pr) + 1;
          j = pair_j(pr);
        }
        const OpT* arow = (isP ? sQ : sK) + (16 * i + l16) * L::LDK;
        const OpT* krow = sKB + (16 * j + l16) * L::LDK;
        f32x4 acc = {0, 0, 0, 0};
#pragma unroll
        for (int m = 0; m < NKP; ++m) {
          auto fa = M::ld_cont(arow, 32 * m, g);
          if (i > j) M::scale_cont(fa, s_tau4 + fac_row(pr) * DK, 32 * m, g);
          M::mma(acc, M::ld_cont(krow, 32 * m, g), fa);
        }
        emit(i, j, isP, acc);
      }
    } else {
      // Exact path: products of exp(g) <= 1 only (see the top of this file).
      // (1b) per quarter and channel: the quarter's decay products.  k times
      // the decay from the quarter start to the token before (Ka) and q times
      // it through the token (Qa) replace k and q; k decayed to the quarter
      // end goes to KB; tau4 is the whole quarter's factor.  The sums over
      // channels of the 6 within-quarter pairs of A and of P are formed here.
      if (qt) {
        float w[12];
#pragma unroll
        for (int x = 0; x < 12; ++x) w[x] = 0.f;
        opv gv[4], kv[4], qv[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int r = 4 * Q + t;
          gv[t] = *reinterpret_cast<const opv*>(sGst + r * DK + c0);
          kv[t] = *reinterpret_cast<const opv*>(sK + r * L::LDK + c0);
          qv[t] = *reinterpret_cast<const opv*>(sQ + r * L::LDK + c0);
        }
        opv ka[4], qa[4], kb[4];
        f32v tau;
#pragma unroll
        for (int e = 0; e < CPT; ++e) {
          float a[4], kx[4], qx[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            a[t] = __expf(static_cast<float>(gv[t][e]));
            kx[t] = static_cast<float>(kv[t][e]);
            qx[t] = static_cast<float>(qv[t][e]);
          }
          float pre = 1.f;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            ka[t][e] = (OpT)(kx[t] * pre);
            pre *= a[t];
            qa[t][e] = (OpT)(qx[t] * pre);
          }
          float suf = 1.f;
#pragma unroll
          for (int t = 3; t >= 0; --t) {
            kb[t][e] = (OpT)(kx[t] * suf);
            suf *= a[t];
          }
          tau[e] = pre;
          // A_rs: decay of s+1 .. r-1; P_rs: of s+1 .. r  (pairs 10 20 21 30 31 32)
          const float a12 = a[1] * a[2], a23 = a[2] * a[3];
          w[0] += kx[1] * kx[0];
          w[1] += kx[2] * kx[0] * a[1];
          w[2] += kx[2] * kx[1];
          w[3] += kx[3] * kx[0] * a12;
          w[4] += kx[3] * kx[1] * a[2];
          w[5] += kx[3] * kx[2];
          w[6] += qx[1] * kx[0] * a[1];
          w[7] += qx[2] * kx[0] * a12;
          w[8] += qx[2] * kx[1] * a[2];
          w[9] += qx[3] * kx[0] * (a12 * a[3]);
          w[10] += qx[3] * kx[1] * a23;
          w[11] += qx[3] * kx[2] * a[3];
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int r = 4 * Q + t;
          *reinterpret_cast<opv*>(sK + r * L::LDK + c0) = ka[t];
          *reinterpret_cast<opv*>(sQ + r * L::LDK + c0) = qa[t];
          *reinterpret_cast<opv*>(sKB + r * L::LDK + c0) = kb[t];
        }
        *reinterpret_cast<f32v*>(s_tau4 + Q * DK + c0) = tau;
#pragma unroll
        for (int x = 0; x < 12; ++x) w[x] = dpp_group_sum<LPQ>(w[x]);
        if (c0 == 0) {
#pragma unroll
          for (int x = 0; x < 12; ++x) s_wq[Q * L::kWQ + x] = w[x];
        }
      }
      lds_barrier();

      // (2a) diagonal blocks: one pass per column quarter S = 0, 1, 2.  Pass S
      // takes the columns of quarter S (k decayed to its end, KB) against the
      // rows of the later quarters R (Ka or Qa) times the decay of the
      // quarters strictly between S and R; the other rows and columns are zero,
      // so the passes add up in one accumulator.
      for (int job = wave; job < 2 * NB; job += kPrepWaves) {
        const bool isP = job >= NB;
        const int i = isP ? job - NB : job;
        const OpT* arow = (isP ? sQ : sK) + (16 * i + l16) * L::LDK;
        const OpT* krow = sKB + (16 * i + l16) * L::LDK;
        const int Rq = l16 >> 2;      // this lane's row quarter and column quarter
        f32x4 acc = {0, 0, 0, 0};
        static_for<3>([&](auto S_) {
          constexpr int S = decltype(S_)::value;
          const float* t1 = s_tau4 + (4 * i + S + 1) * DK;
          const float* t2 = s_tau4 + (4 * i + (S + 2 < 4 ? S + 2 : 3)) * DK;
#pragma unroll
          for (int m = 0; m < NKP; ++m) {
            typename M::frag fk = Rq == S ? M::ld_cont(krow, 32 * m, g) : M::zero();
            typename M::frag fa = Rq > S ? M::ld_cont(arow, 32 * m, g) : M::zero();
            if constexpr (S < 2) M::scale_cont2(fa, t1, Rq >= S + 2, t2, S < 1 && Rq >= S + 3, 32 * m, g);
            M::mma(acc, fk, fa);
          }
        });
        emit(i, i, isP, acc);
      }
      lds_barrier();

      // (2b) from quarters to blocks: Ka, Qa times the decay of the earlier
      // quarters of their block, KB times that of the later ones; the record's
      // chunk-referenced operands K = k exp(Gx), Q = q exp(G) and
      // F = k exp(G_last - G); exp(G_last) per channel; and D, the decay of the
      // blocks strictly between two blocks i - j >= 2 apart.
      if (qt) {
        const int blk = Q >> 2;
        f32v t16[NB], cqp = 1.f, cqs = 1.f;
#pragma unroll
        for (int b2 = 0; b2 < NB; ++b2) t16[b2] = 1.f;
#pragma unroll
        for (int q2 = 0; q2 < NQ; ++q2) {
          const f32v t = *reinterpret_cast<const f32v*>(s_tau4 + q2 * DK + c0);
          t16[q2 >> 2] *= t;
          if ((q2 >> 2) == blk && q2 < Q) cqp *= t;
          if ((q2 >> 2) == blk && q2 > Q) cqs *= t;
        }
        f32v cb = 1.f, ca = 1.f, all = 1.f;
#pragma unroll
        for (int b2 = 0; b2 < NB; ++b2) {
          if (b2 < blk) cb *= t16[b2];
          if (b2 > blk) ca *= t16[b2];
          all *= t16[b2];
        }
        if (Q == 0) {
          *reinterpret_cast<f32v*>(rvec + R::vDecC + c0) = all;
#pragma unroll
          for (int i2 = 2; i2 < NB; ++i2) {
            f32v dd = 1.f;
#pragma unroll
            for (int j2 = i2 - 2; j2 >= 0; --j2) {
              dd *= t16[j2 + 1];
              *reinterpret_cast<f32v*>(s_D + L::ddslot(i2, j2) * DK + c0) = dd;
            }
          }
        }
        // (s_D overlays the within-quarter sums, whose last reader was (2a))
        const f32v fkq = cqp * cb, ff = cqs * ca;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int r = 4 * Q + t;
          const opv ka = *reinterpret_cast<const opv*>(sK + r * L::LDK + c0);
          const opv qa = *reinterpret_cast<const opv*>(sQ + r * L::LDK + c0);
          const opv kb = *reinterpret_cast<const opv*>(sKB + r * L::LDK + c0);
          opv ka16, qa16, kb16;
          float xk[CPT], xq[CPT], xf[CPT];
#pragma unroll
          for (int e = 0; e < CPT; ++e) {
            const float k1 = static_cast<float>(ka[e]), q1 = static_cast<float>(qa[e]);
            const float b1 = static_cast<float>(kb[e]);
            ka16[e] = (OpT)(k1 * cqp[e]);
            qa16[e] = (OpT)(q1 * cqp[e]);
            kb16[e] = (OpT)(b1 * cqs[e]);
            xk[e] = k1 * fkq[e];
            xq[e] = q1 * fkq[e];
            xf[e] = b1 * ff[e];
          }
          *reinterpret_cast<opv*>(sK + r * L::LDK + c0) = ka16;
          *reinterpret_cast<opv*>(sQ + r * L::LDK + c0) = qa16;
          *reinterpret_cast<opv*>(sKB + r * L::LDK + c0) = kb16;
          if constexpr (CPT % 4 == 0) {
            put_perm<OpT, R::PPRK>(rec + R::oK, r, c0, xk);
            put_perm<OpT, R::PPRK>(rec + R::oQ, r, c0, xq);
            put_perm<OpT, R::PPRK>(rec + R::oF, r, c0, xf);
          } else {
#pragma unroll
            for (int e = 0; e < CPT; ++e) {
              const int off = swz_off<R::PPRK>(r, perm_pos(c0 + e) * static_cast<int>(sizeof(OpT)));
              *reinterpret_cast<OpT*>(rec + R::oK + off) = (OpT)xk[e];
              *reinterpret_cast<OpT*>(rec + R::oQ + off) = (OpT)xq[e];
              *reinterpret_cast<OpT*>(rec + R::oF + off) = (OpT)xf[e];
            }
          }
        }
      }
      lds_barrier();

      // (2c) off-diagonal blocks i > j: the rows decayed from their block's
      // start (Ka, Qa) times D, against k decayed to the end of block j (KB)
      constexpr int NOFF = NB * (NB - 1) / 2;
      for (int job = wave; job < 2 * NOFF; job += kPrepWaves) {
        const bool isP = job >= NOFF;
        const int pr = isP ? job - NOFF : job;
        const int i = pair_i(pr) + 1, j = pair_j(pr);    // pairs of the strictly lower triangle
        const OpT* arow = (isP ? sQ : sK) + (16 * i + l16) * L::LDK;
        const OpT* krow = sKB + (16 * j + l16) * L::LDK;
        const float* dv = s_D + L::ddslot(i > j + 1 ? i : 2, i > j + 1 ? j : 0) * DK;
        f32x4 acc = {0, 0, 0, 0};
#pragma unroll
        for (int m = 0; m < NKP; ++m) {
          auto fa = M::ld_cont(arow, 32 * m, g);
          if (i > j + 1) M::scale_cont(fa, dv, 32 * m, g);
          M::mma(acc, M::ld_cont(krow, 32 * m, g), fa);
        }
        emit(i, j, isP, acc);
    }
    }
  }
  lds_barrier();

  // ============ phase 3: T = (I + A)^-1 (fp32) ============
  // diagonal blocks of T into their region, over tiles the Gram has now
  // finished reading
  if constexpr (!chan) {
    if (wave == 0 && g < NB) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sTm[(16 * g + r) * L::LF + 16 * g + l16] = xd[r];
    }
  } else if (wave == 0) {
    // per-channel decay: after the Gram, lane -> (block, column)
    if (g < NB) {
      float x[16];
      diag_inverse(g, l16, x);
#pragma unroll
      for (int r = 0; r < 16; ++r) sTm[(16 * g + r) * L::LF + 16 * g + l16] = x[r];
    }
  }
  if (wave != 0) {
    // meanwhile the other waves zero P above the block diagonal (never
    // produced by the Gram)
    constexpr int VE = 16 / sizeof(OpT);
    constexpr int RowV = R::NCOL / VE;       // 16-byte pieces per P row
    for (int idx = tid - 64; !R::kRawK && idx < C * RowV; idx += kPrepThreads - 64) {
      const int r = idx / RowV, s0 = (idx % RowV) * VE;
      if ((s0 >> 4) > (r >> 4)) {
        float x[VE];
#pragma unroll
        for (int e = 0; e < VE; ++e) x[e] = 0.f;
        put_perm<OpT, R::PPRC>(rec + R::oP, r, s0, x);
      }
    }
  }
  lds_barrier();
#pragma unroll
  for (int d = 1; d < NB; ++d) {
    // blocks on diagonal d: T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj, on waves 1..
    const int j = wave - 1, i = j + d;
    if (wave >= 1 && i < NB) {
      // every operand read first (one wait), then the MFMA chain
      f32x4 a4[NB], t4;
      float bv[NB][4];
#pragma unroll
      for (int kk = 0; kk < d; ++kk) {
        a4[kk] = *reinterpret_cast<const f32x4*>(sAm + (16 * i + l16) * L::LF + 16 * (j + kk) + 4 * g);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) bv[kk][jj] = sTm[(16 * (j + kk) + 4 * g + jj) * L::LF + 16 * j + l16];
      }
      t4 = *reinterpret_cast<const f32x4*>(sTm + (16 * i + l16) * L::LF + 16 * i + 4 * g);
      __builtin_amdgcn_sched_barrier(0);
      f32x4 X = {0, 0, 0, 0};
#pragma unroll
      for (int kk = 0; kk < d; ++kk) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) X = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[kk][jj], bv[kk][jj], X, 0, 0, 0);
      }
      f32x4 Y = {0, 0, 0, 0};
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) Y = __builtin_amdgcn_mfma_f32_16x16x4f32(t4[jj], X[jj], Y, 0, 0, 0);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) sTm[(16 * i + 4 * g + jj) * L::LF + 16 * j + l16] = -Y[jj];
    }
    lds_barrier();
  }

  // ============ record: T diag(beta), zero above the block diagonal ============
  {
    constexpr int VE = 16 / sizeof(OpT);
    constexpr int RowV = R::NCOL / VE;
    for (int idx = tid; idx < C * RowV; idx += kPrepThreads) {
      const int r = idx / RowV, s0 = (idx % RowV) * VE;
      float x[VE];
      const bool upper = (s0 >> 4) > (r >> 4);
#pragma unroll
      for (int e = 0; e < VE; ++e) x[e] = upper ? 0.f : sTm[r * L::LF + s0 + e] * s_bt[s0 + e];
      put_perm<OpT, R::PPRC>(rec + R::oTu, r, s0, x);
    }
  }
}

// ------------------------------------------------------------ state kernel --

// Wait until this wave's global loads (the LDS copies included) have landed.
__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// Wait until at most N of this wave's global loads are outstanding (loads
// complete in issue order: all but the last N have landed).
template <int N>
__device__ __forceinline__ void wait_vm_keep() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}
// Wait until this wave's LDS reads have returned.
__device__ __forceinline__ void wait_lgkm() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// MFMA fragments from a chunk record in LDS (tiles with rows of 16-byte
// pieces, elements in perm_pos order, swizzled).  The swizzle repeats every
// 16 rows, so every fragment address is one of a few per-lane offsets,
// computed once, plus a compile-time displacement (row block, k step, tile,
// buffer).
//   kq(tile, rt, m)    Q/K/F rows 16 rt + l16, k = 32 m + {4g..4g+3, 16+4g..}
//   cc(tile, rt, m)    the same for the [C][NCOL] tiles Tu and P
//   tok(tile, m, t, hi) the transposed operand: channel 16 t + l16 at tokens
//                      32 m + 4g + j and (hi) 32 m + 16 + 4g + j
template <int DK, int C, typename OpT> struct RecFrags;
template <int DK, int C> struct RecFrags<DK, C, _Float16> {
  using R = RecLayout<DK, C, 2, false>;
  static constexpr int RowK = R::PPRK * 16, RowC = R::PPRC * 16;
  int kqo[DK / 32], cco[R::NCOL / 32], toko[DK / 32];
  __device__ void init(int g, int l16) {
#pragma unroll
    for (int m = 0; m < DK / 32; ++m) kqo[m] = swz_off<R::PPRK>(l16, 2 * (32 * m + 8 * g));
#pragma unroll
    for (int m = 0; m < R::NCOL / 32; ++m) cco[m] = swz_off<R::PPRC>(l16, 2 * (32 * m + 8 * g));
#pragma unroll
    for (int a = 0; a < DK / 32; ++a)
      toko[a] = swz_off<R::PPRK>(4 * g + (l16 >> 2), 2 * perm_pos(32 * a + 4 * (l16 & 3)));
  }
  __device__ f16x8 kq(const unsigned char* tile, int rt, int m) const {
    return *reinterpret_cast<const f16x8*>(tile + kqo[m] + 16 * rt * RowK);
  }
  __device__ f16x8 cc(const unsigned char* tile, int rt, int m) const {
    return *reinterpret_cast<const f16x8*>(tile + cco[m] + 16 * rt * RowC);
  }
  __device__ f16x8 tok(const unsigned char* tile, int m, int t, bool hi) const {
    const unsigned char* at = tile + toko[t >> 1] + 32 * m * RowK + 8 * (t & 1);
    const f16x4 lo = ld_tr16(reinterpret_cast<const _Float16*>(at));
    const f16x4 up = hi ? ld_tr16(reinterpret_cast<const _Float16*>(at + 16 * RowK)) : f16x4{0, 0, 0, 0};
    return __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7);
  }
};
template <int DK, int C> struct RecFrags<DK, C, float> {
  using R = RecLayout<DK, C, 4, false>;
  using frag = Mma<float>::frag;
  int g, l16;
  __device__ void init(int g_, int l16_) { g = g_; l16 = l16_; }
  template <int PPR>
  __device__ frag perm(const unsigned char* tile, int r, int m) const {
    frag f;
    f.lo = *reinterpret_cast<const f32x4*>(tile + swz_off<PPR>(r, 4 * (32 * m + 8 * g)));
    f.hi = *reinterpret_cast<const f32x4*>(tile + swz_off<PPR>(r, 4 * (32 * m + 8 * g + 4)));
    return f;
  }
  __device__ frag kq(const unsigned char* tile, int rt, int m) const { return perm<R::PPRK>(tile, 16 * rt + l16, m); }
  __device__ frag cc(const unsigned char* tile, int rt, int m) const { return perm<R::PPRC>(tile, 16 * rt + l16, m); }
  __device__ frag tok(const unsigned char* tile, int m, int t, bool hi) const {
    frag f;
    const int b = 4 * perm_pos(16 * t + l16);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f.lo[j] = *reinterpret_cast<const float*>(tile + swz_off<R::PPRK>(32 * m + 4 * g + j, b));
      f.hi[j] = hi ? *reinterpret_cast<const float*>(tile + swz_off<R::PPRK>(32 * m + 16 + 4 * g + j, b)) : 0.f;
    }
    return f;
  }
};

// Raw buffer resource (V#) over `bytes` bytes at `base`, dword data.
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 rsrc(const void* base, int bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return i32x4{static_cast<int32_t>(a & 0xffffffffu), static_cast<int32_t>((a >> 32) & 0xffffu), bytes,
               0x00020000};
}
// The LDS byte address of a pointer into LDS.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void*)(p)));
}
// Asynchronous 16-byte copy global -> LDS (buffer_load_dwordx4 ... lds):
// lane i of the wave writes LDS byte address m0 + 16 i (m0 wave-uniform),
// reading the buffer at voff (per lane) + soff (uniform).  Written as
// assembly so that the compiler does not wait for the copy before unrelated
// LDS reads; the caller waits (wait_vm) and synchronises before
// the copied data is read.
__device__ __forceinline__ void dma16_buf(i32x4 rs, uint32_t m0, int voff, int soff) {
  // every scalar operand is wave-uniform; make that explicit so each lands in
  // an SGPR, and leave M0 as it was found
  const i32x4 r = i32x4{__builtin_amdgcn_readfirstlane(rs[0]), __builtin_amdgcn_readfirstlane(rs[1]),
                        __builtin_amdgcn_readfirstlane(rs[2]), __builtin_amdgcn_readfirstlane(rs[3])};
  int saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, %4 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(__builtin_amdgcn_readfirstlane(m0)), "v"(voff), "s"(r), "s"(__builtin_amdgcn_readfirstlane(soff))
      : "memory");
}

// L2 prefetch: a 4-byte load per lane (buffer_load_dword ... lds) whose data
// lands in a dummy LDS slot at m0 (lane i at m0 + 4 i), so no register waits
// for it; its purpose is the line it brings into the L2.  Offsets outside the
// buffer's range read nothing.
__device__ __forceinline__ void touch_buf(i32x4 rs, uint32_t m0, int voff) {
  const i32x4 r = i32x4{__builtin_amdgcn_readfirstlane(rs[0]), __builtin_amdgcn_readfirstlane(rs[1]),
                        __builtin_amdgcn_readfirstlane(rs[2]), __builtin_amdgcn_readfirstlane(rs[3])};
  int saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(__builtin_amdgcn_readfirstlane(m0)), "v"(voff), "s"(r)
      : "memory");
}

// State-kernel workgroup: DVS/16 owner waves that compute, and as many
// helper waves that copy the next chunk into LDS, so the owners never wait to
// issue a copy.
template <int DVS> constexpr int state_waves() { return DVS / 16 + state_helpers<DVS>(); }

template <int DK, int DVS, int C, typename In, int DECAY>
__global__ __launch_bounds__(64 * state_waves<DVS>(), state_waves<DVS>() > 4 ? 2 : 1)
void state_kernel(StateParams p) {
  using OpT = typename OpOf<In>::T;
  using M = Mma<OpT>;
  constexpr bool chan = DECAY == DECAY_CHANNEL;
  constexpr bool headdecay = DECAY == DECAY_HEAD;
  constexpr int AB = sizeof(In);               // activation bytes
  using L = StateLayout<DK, DVS, C, sizeof(OpT), AB, chan>;
  using R = RecLayout<DK, C, sizeof(OpT), chan>;
  constexpr int NB = C / 16;
  constexpr int NKT = DK / 16;               // 16-row tiles of the state
  constexpr int NKP = DK / 32;               // 32-wide k steps over the key dim
  constexpr int NOWN = DVS / 16;             // waves that own state columns
  constexpr int NH = (NB + 1) / 2;           // 32-wide k steps over the chunk's tokens
  // 16-byte copies per chunk, each helper wave issuing its share: (raw rows)
  // the q and k rows, the record, the value rows
  constexpr bool rawk = R::kRawK;
  constexpr int nRecI = static_cast<int>(L::kRecLds / 1024);   // whole slots (image padded)
  constexpr int nVal = C * L::PPRV, nValI = (nVal + 63) / 64;
  constexpr int nQK = rawk ? C * R::PPRK : 0, nQKI = nQK / 64;
  constexpr int NHELP = state_helpers<DVS>();  // helper waves (they issue every copy)
  constexpr int NPF = L::kNPF;                // P operand fragments (raw rows: formed by the helpers)
  constexpr int NBLK = NB * (NB + 1) / 2;     // P's lower-triangular 16 x 16 blocks
  constexpr int kStThreads = 64 * state_waves<DVS>();
  constexpr int kSlotsR = nRecI / NHELP, kSlotsV = (nValI + NHELP - 1) / NHELP;
  static_assert(nRecI % NHELP == 0, "record slots shared evenly");
  constexpr int kSlotsQ = rawk ? (nQKI + NHELP - 1) / NHELP : 0;
  static_assert(DVS % 16 == 0 && NOWN + NHELP == state_waves<DVS>(), "slice width");
  static_assert(L::PPRV >= 1, "value rows hold whole 16-byte pieces");
  static_assert(nQK % 64 == 0, "k copies fill whole instructions");
  // L2 prefetch loads per helper and chunk (64-byte lines; sized for one
  // slice per head, the most a slice prefetches): the record's and (raw rows)
  // the q and k rows' share of this slice, and its own value rows
  constexpr int kLinesRec = static_cast<int>((R::gBytes + 63) / 64);
  constexpr int kLinesQK = rawk ? C * DK * AB / 64 : 0;       // per tensor
  constexpr int kLPV = (DVS * AB + 63) / 64;                  // lines per value row
  constexpr int kPfR = (kLinesRec + 64 * NHELP - 1) / (64 * NHELP);
  constexpr int kPfQ = (kLinesQK + 64 * NHELP - 1) / (64 * NHELP);
  constexpr int kPfV = (C * kLPV + 64 * NHELP - 1) / (64 * NHELP);
  // (with raw rows the record is small and the owners bound the step: no prefetch)
  constexpr bool kPrefetch = !rawk;
  static_assert(!kPrefetch || L::kTouch == 256, "the prefetch slot");
  constexpr int kPf = kPrefetch ? kPfR + 2 * kPfQ + kPfV : 0;   // the most a helper issues per chunk
  int npf = 0;                                  // prefetch loads of the last issue

  extern __shared__ __align__(256) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  const int b = head / H, h = head % H;   // (packed input: b is the sequence)
  const int n0 = slice * DVS;   // first value column of this slice
  const In* gv = static_cast<const In*>(p.v);
  const In* gq = static_cast<const In*>(p.q);
  const In* gk = static_cast<const In*>(p.k);
  const unsigned char* rec0;                 // the first chunk's record
  long seq0;                                 // first token of this launch
  int Trem;                                  // tokens from there to the sequence end
  int nchunks;
  if (p.cu) {
    rec0 = p.ws + (static_cast<size_t>(h) * p.nchunks + p.cb[b]) * R::gBytes;
    seq0 = p.cu[b];
    Trem = p.cu[b + 1] - p.cu[b];
    nchunks = p.cb[b + 1] - p.cb[b];
  } else {
    rec0 = p.ws + static_cast<size_t>(head) * p.nchunks * R::gBytes;
    seq0 = static_cast<long>(b) * T + static_cast<long>(p.c0) * C;
    Trem = T - p.c0 * C;
    nchunks = p.nchunks;
  }
  const int rowV = H * DV * AB;              // bytes between consecutive tokens of v
  const int rowK = p.Hk * DK * AB;           // ... of q and k (q/k heads)
  const int hk = qk_head(h, p.hk_magic);     // the q/k head of value head h
  const int rowO = H * DV * 4;               // ... and of o

  RecFrags<DK, C, OpT> fr;
  fr.init(g, l16);
  // value rows 4g + jj (+16 rt) at this lane's column: bf16 rows are read
  // transposed (one read per 16-row block), fp32 rows one element at a time
  constexpr int RowV = L::PPRV * 16;
  const int vtr = swzv_off<L::PPRV>(4 * g + (l16 >> 2), (16 * wave + 4 * (l16 & 3)) * AB);
  int vo[4];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) vo[jj] = swzv_off<L::PPRV>(4 * g + jj, (16 * wave + l16) * AB);

  // ---- the state slice: owner wave w keeps value columns n0 + 16w .. +15 ----
  const bool owner = wave < NOWN;
  const int hw = wave - NOWN;                // helper index (helper waves)
  // Per-lane copy offsets of a helper wave, the same for every chunk: value
  // piece of slot s is row vr[s] (-1: past the value rows, no copy), at byte
  // voff[s] from the chunk's first value element; q and k piece of slot s is
  // row kr[s], at byte kvo[s] from the chunk's first q or k element, landing
  // at the swizzled position of the Q or K tile.
  int vr[kSlotsV], voff[kSlotsV];
#pragma unroll
  for (int sv = 0; sv < kSlotsV; ++sv) {
    const int piece = (sv * NHELP + hw) * 64 + lane;
    const int r = piece / L::PPRV, q = piece % L::PPRV;
    vr[sv] = piece < nVal ? r : -1;
    voff[sv] = r * rowV + (q ^ swzv<L::PPRV>(r)) * 16;
  }
  int kr[kSlotsQ > 0 ? kSlotsQ : 1], kvo[kSlotsQ > 0 ? kSlotsQ : 1];
#pragma unroll
  for (int sq = 0; sq < kSlotsQ; ++sq) {
    const int w = (sq * NHELP + hw) * 64 + lane;   // piece of the K tile
    const int r = w / R::PPRK, pos = w % R::PPRK;
    kr[sq] = r;
    kvo[sq] = r * rowK + (pos ^ swz<R::PPRK>(r)) * 16;
  }

  // Copy chunk c into LDS buffer `buf` (helper waves, asynchronous; slot s of
  // a helper is one 1 KiB copy instruction).  Rows past the sequence end copy
  // the chunk's row 0 instead (finite data; their products only meet zero
  // rows of T and P, and value rows are cleared once the copies land).
  const uint32_t lds0 = lds_addr(smem);
  // part 1: (raw rows) the q and k rows, part 2: the record and the value
  // rows, 0: both
  auto issue = [&](int c, unsigned char* dstp, auto part_tag) __attribute__((always_inline)) {
    constexpr int part = decltype(part_tag)::value;
    const uint32_t dst = lds0 + static_cast<uint32_t>(dstp - smem);
    const int t0 = c * C, Lc = min(C, Trem - t0);
    if constexpr (part != 2) {
      if constexpr (rawk) {
        const long e0 = ((seq0 + t0) * p.Hk + hk) * static_cast<long>(DK);
        const int nb = (Lc - 1) * rowK + DK * AB;
        const i32x4 rk = rsrc(gk + e0, nb), rq = rsrc(gq + e0, nb);
#pragma unroll
        for (int sq = 0; sq < kSlotsQ; ++sq) {
          const int j = sq * NHELP + hw;
          if (nQKI % NHELP == 0 || j < nQKI) {
            const int off = kr[sq] < Lc ? kvo[sq] : 0;
            dma16_buf(rk, dst + R::oK + j * 1024, off, 0);
            dma16_buf(rq, dst + R::oQ + j * 1024, off, 0);
          }
        }
      }
    }
    if constexpr (part == 1) return;
    const i32x4 rr = rsrc(rec0 + static_cast<size_t>(c) * R::gBytes, static_cast<int>(R::gBytes));
    // (the record's LDS image is padded to whole slots of every helper;
    // pieces past the record read as zero through the buffer's range check)
#pragma unroll
    for (int sl = 0; sl < kSlotsR; ++sl) {
      const int j = sl * NHELP + hw;
      dma16_buf(rr, dst + R::gOff + j * 1024, j * 1024 + lane * 16, 0);
    }
    {
      const i32x4 rv =
          rsrc(gv + ((seq0 + t0) * H + h) * static_cast<long>(DV) + n0, (Lc - 1) * rowV + DVS * AB);
#pragma unroll
      for (int sv = 0; sv < kSlotsV; ++sv) {
        const int j = sv * NHELP + hw;
        if ((nVal % (64 * NHELP) == 0 || (j < nValI && vr[sv] >= 0)))
          dma16_buf(rv, dst + L::oV + j * 1024, vr[sv] < Lc ? voff[sv] : 0, 0);
      }
    }
    // Prefetch chunk c + 1 into the L2, one step before its copy: this
    // slice's share of the lines every slice of the head copies (the record,
    // and with raw rows the q and k rows), and its own value rows.  These are
    // the last loads this helper issues before its wait (finish), which leaves
    // them in flight; npf counts them.  Lanes past the share repeat a line of
    // it (no load leaves the buffers).
    npf = 0;
    if (kPrefetch && c + 1 < nchunks) {
      const int cn = c + 1, tn = cn * C, Ln = min(C, Trem - tn);
      const uint32_t tslot = lds0 + static_cast<uint32_t>(L::oTouch);
      const int shareR = min((kLinesRec + p.nsl - 1) / p.nsl, kLinesRec - slice * ((kLinesRec + p.nsl - 1) / p.nsl));
      const int firstR = slice * ((kLinesRec + p.nsl - 1) / p.nsl);
      const i32x4 rr2 = rsrc(rec0 + static_cast<size_t>(cn) * R::gBytes, static_cast<int>(R::gBytes));
      const int nR = shareR > 0 ? (shareR + 64 * NHELP - 1) / (64 * NHELP) : 0;
      for (int i = 0; i < nR; ++i) {
        const int li = (i * NHELP + hw) * 64 + lane;
        touch_buf(rr2, tslot, (firstR + (li < shareR ? li : 0)) * 64);
      }
      npf += nR;
      if constexpr (rawk && kPrefetch) {
        const long e1 = ((seq0 + tn) * p.Hk + hk) * static_cast<long>(DK);
        const i32x4 rk2 = rsrc(gk + e1, (Ln - 1) * rowK + DK * AB), rq2 = rsrc(gq + e1, (Ln - 1) * rowK + DK * AB);
        constexpr int LPK = DK * AB / 64;   // lines per q or k row
        const int lines = Ln * LPK, per = (lines + p.nsl - 1) / p.nsl;
        const int firstQ = slice * per, shareQ = min(per, lines - firstQ);
        const int nQ = shareQ > 0 ? (shareQ + 64 * NHELP - 1) / (64 * NHELP) : 0;
        for (int i = 0; i < nQ; ++i) {
          const int li = (i * NHELP + hw) * 64 + lane, line = firstQ + (li < shareQ ? li : 0);
          const int off = (line / LPK) * rowK + (line % LPK) * 64;
          touch_buf(rk2, tslot, off);
          touch_buf(rq2, tslot, off);
        }
        npf += 2 * nQ;
      }
      const i32x4 rv2 = rsrc(gv + ((seq0 + tn) * H + h) * static_cast<long>(DV) + n0, (Ln - 1) * rowV + DVS * AB);
      const int linesV = Ln * kLPV, nV = (linesV + 64 * NHELP - 1) / (64 * NHELP);
      for (int i = 0; i < nV; ++i) {
        const int li = (i * NHELP + hw) * 64 + lane, line = li < linesV ? li : 0;
        touch_buf(rv2, tslot, (line / kLPV) * rowV + (line % kLPV) * 64);
      }
      npf += nV;
    }
  };
  // After the copy of chunk c into `buf` has landed: value rows past the
  // sequence end read as zero (each helper clears the pieces it copied).
  auto zero_tail = [&](int c, unsigned char* buf) __attribute__((always_inline)) {
    const int Lc = min(C, Trem - c * C);
    if (!owner && Lc < C) {
      unsigned char* dst = buf + L::oV;
#pragma unroll
      for (int sv = 0; sv < kSlotsV; ++sv) {
        const int j = sv * NHELP + hw;
        if ((nVal % (64 * NHELP) == 0 || (j < nValI && vr[sv] >= 0)) && vr[sv] >= Lc)
          *reinterpret_cast<u32x4*>(dst + j * 1024 + lane * 16) = u32x4{0, 0, 0, 0};
      }
    }
  };
  auto finish = [&](int c, unsigned char* buf) __attribute__((always_inline)) {
    // the copies have landed; the npf prefetch loads after them may not have
    static_for<kPf + 1>([&](auto n_) {
      constexpr int n = decltype(n_)::value;
      if (npf == n) wait_vm_keep<n>();
    });
    if (npf > kPf) wait_vm();
    zero_tail(c, buf);
  };

  const int ncol = n0 + 16 * wave + l16;   // this lane's value column (owner waves)
  // Row j of lane group g of tile t holds key channel srow(t, j).  With the
  // record's perm_pos order the tiles are plain 16-row bands; with raw K
  // (natural order Q and K rows) tiles 2m and 2m+1 interleave the channels of
  // the 32-channel block m in fours, so that a lane's 8 operand elements are
  // 8 consecutive channels in both layouts.
  auto srow = [&](int t, int j) {
    return rawk ? 32 * (t >> 1) + 8 * g + 4 * (t & 1) + j : 16 * t + 4 * g + j;
  };
  // element (key row, this lane's column) of the initial / final state
  const long sbase = (static_cast<long>(b) * H + h) * DK * DV;
  auto sidx = [&](int row) {
    return sbase + (p.vfirst ? static_cast<long>(ncol) * DK + row : static_cast<long>(row) * DV + ncol);
  };
  f32x4 S[NKT];
#pragma unroll
  for (int t = 0; t < NKT; ++t) {
    S[t] = f32x4{0, 0, 0, 0};
    if (owner && p.init) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        S[t][j] = p.init[sidx(srow(t, j))];
    }
  }

  // Raw rows (see StateLayout): the helpers form P's operand fragments and
  // q's row factors, and flag each chunk's.
  constexpr bool hp = L::kHelperP;
  static_assert(hp == rawk, "raw rows go with the helper-formed P");
  int* pflags = reinterpret_cast<int*>(smem + L::oFlags);   // helper h's P of chunk c written: c + 1
  float* sfq = reinterpret_cast<float*>(smem + L::oFQ);     // q's row factor per token of the chunk
  if constexpr (hp) {
    if (!owner && lane == 0) pflags[hw] = 0;
    // the fragments' halves above the diagonal (column block ib + 1 of an
    // even row block ib) stay zero
    if (hw == 0) {
#pragma unroll
      for (int ib = 0; ib < NB; ib += 2)
        *reinterpret_cast<f16x4*>(smem + L::oPF + pf_n(ib, ib / 2) * 1024 + lane * 16 + 8) = f16x4{0, 0, 0, 0};
    }
  }

  if (nchunks > 0) {
    if (!owner) issue(0, smem, std::integral_constant<int, 0>{});
    if (!owner) finish(0, smem);
  }
  lds_barrier();

  // Output rows of a chunk (without raw rows stored at the start of the next
  // one, so that the stores wait for nothing)
  f32x4 Oprev[NB];
  const int obyte = 16 * wave * 4 + 4 * g * 4;   // this lane's column bytes within a row of o (owners)
  auto store_out = [&](int c) {
    const int t0 = c * C, Lc = min(C, Trem - t0);
    unsigned char* ob = reinterpret_cast<unsigned char*>(p.o + ((seq0 + t0) * H + h) * static_cast<long>(DV) + n0);
#pragma unroll
    for (int rt = 0; rt < NB; ++rt) {
      const int r = 16 * rt + l16;
      if (r < Lc) *reinterpret_cast<f32x4*>(ob + r * rowO + obyte) = Oprev[rt];
    }
  };
  // One chunk step on LDS buffer CUR (a compile-time constant, so every LDS
  // address below is a per-lane base plus an immediate), for an owner or a
  // helper wave (a compile-time choice: the two kinds of wave run separate
  // loops, so neither holds the other's registers).
  auto step = [&](auto cur_tag, auto own_tag, int c) {
    constexpr int cur = decltype(cur_tag)::value;
    constexpr bool own = decltype(own_tag)::value;
    // the helpers copy the next chunk into the other buffer meanwhile
    const bool pre = L::NBUF == 2 && c + 1 < nchunks;

    if constexpr (own) {
      const unsigned char* bq = smem + cur * L::kBuf;
      const unsigned char* sQ = bq + R::oQ;
      const unsigned char* sK = bq + R::oK;
      const unsigned char* sKF = bq + R::oF;
      const unsigned char* sTu = bq + R::oTu;
      const unsigned char* sP = bq + R::oP;
      const unsigned char* sV = bq + L::oV;
      const float* svec = reinterpret_cast<const float*>(bq + R::oVec);

      if (!rawk && c > 0) store_out(c - 1);
      // Raw rows: the products with q and k run in bf16 (their rows as given,
      // S0 and D in two bf16 parts, or S0 in one for K S0); the row factors
      // are in the per-token vectors and FQ.
      [[maybe_unused]] typename M::frag Sf[NKP];
      [[maybe_unused]] bf16x8 Sb[NKP];
#pragma unroll
      for (int m = 0; m < NKP; ++m) {
        if constexpr (rawk) Sb[m] = bf_from_acc(S[2 * m], S[2 * m + 1]);
        else Sf[m] = M::from_acc(S[2 * m], S[2 * m + 1]);
      }
      // K S0 and S0^T Q^T: both read only S0, so their products interleave
      f32x4 Xl[NB], Ol[NB];
      if constexpr (rawk) {
        // every operand first, then the products with each accumulator's
        // successive steps NB products apart (S0 in two bf16 parts for the
        // output, the low part into Ol2)
        bf16x8 fqb[NB][NKP], fkb[NB][NKP];
        f32x4 Ol2[NB];
#pragma unroll
        for (int rt = 0; rt < NB; ++rt) {
#pragma unroll
          for (int m = 0; m < NKP; ++m) {
            fkb[rt][m] = __builtin_bit_cast(bf16x8, fr.kq(sK, rt, m));
            fqb[rt][m] = __builtin_bit_cast(bf16x8, fr.kq(sQ, rt, m));
          }
          Xl[rt] = Ol[rt] = Ol2[rt] = f32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int m = 0; m < NKP; ++m) {
          const bf16x8 sl = bf_lo(S[2 * m], S[2 * m + 1], Sb[m]);
#pragma unroll
          for (int rt = 0; rt < NB; ++rt) mma_bf(Xl[rt], fkb[rt][m], Sb[m]);
#pragma unroll
          for (int rt = 0; rt < NB; ++rt) mma_bf(Ol[rt], Sb[m], fqb[rt][m]);
#pragma unroll
          for (int rt = 0; rt < NB; ++rt) mma_bf(Ol2[rt], sl, fqb[rt][m]);
        }
#pragma unroll
        for (int rt = 0; rt < NB; ++rt) Ol[rt] += Ol2[rt];
      } else {
#pragma unroll
        for (int rt = 0; rt < NB; ++rt) {
          typename M::frag fqf[NKP], fkf[NKP];
#pragma unroll
          for (int m = 0; m < NKP; ++m) {
            fkf[m] = fr.kq(sK, rt, m);
            fqf[m] = fr.kq(sQ, rt, m);
          }
          Xl[rt] = Ol[rt] = f32x4{0, 0, 0, 0};
#pragma unroll
          for (int m = 0; m < NKP; ++m) {
            M::mma(Xl[rt], fkf[m], Sf[m]);
            M::mma(Ol[rt], Sf[m], fqf[m]);
          }
        }
      }
      // X = V - (K * exp(Gx)) S0
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) {
        float vv[4];
        if constexpr (AB == 2) {
          typedef short s4 __attribute__((ext_vector_type(4)));
          const s4 tv = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) s4*)(sV + vtr + 16 * rt * RowV));
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) vv[jj] = bf16_to_f32(static_cast<uint16_t>(tv[jj]));
        } else {
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            vv[jj] = act<In>::load1(reinterpret_cast<const In*>(sV + vo[jj] + 16 * rt * RowV));
        }
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int r = 16 * rt + 4 * g + jj;
          float ks = Xl[rt][jj];
          if (headdecay || rawk) ks *= svec[R::vEGx + r];
          Xl[rt][jj] = vv[jj] - ks;
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
#pragma unroll
        for (int m = 0; m <= rt / 2; ++m) M::mma(Dl[rt], fr.cc(sTu, rt, m), Xf[m]);
      }
      typename M::frag Df[NH];
#pragma unroll
      for (int m = 0; m < NH; ++m)
        Df[m] = M::from_acc(Dl[2 * m], 2 * m + 1 < NB ? Dl[2 * m + 1] : f32x4{0, 0, 0, 0});
      // O^T = S0^T (Q * exp(G))^T + D^T P^T; raw rows: q's row factor on
      // the first term, P from the helpers (after the state step, which
      // does not need it)
      auto form_out = [&]() {
        if constexpr (rawk) {
#pragma unroll
          for (int h2 = 0; h2 < NHELP; ++h2) {
            while (__hip_atomic_load(&pflags[h2], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < c + 1)
              __builtin_amdgcn_s_sleep(1);
          }
        }
#pragma unroll
        for (int rt = 0, n = 0; rt < NB; ++rt) {
          float f = headdecay ? svec[R::vEG + 16 * rt + l16] : 1.f;
          if constexpr (rawk) f *= sfq[16 * rt + l16];
          if (headdecay || rawk) Ol[rt] *= f;
#pragma unroll
          for (int m = 0; m <= rt / 2; ++m, ++n) {
            if constexpr (rawk)
              M::mma(Ol[rt], Df[m], *reinterpret_cast<const typename M::frag*>(smem + L::oPF + n * 1024 + lane * 16));
            else
              M::mma(Ol[rt], Df[m], fr.cc(sP, rt, m));
          }
        }
      };
      if constexpr (!rawk) form_out();
      // S <- exp(G_last) S0 + KY^T D, KY = K * exp(G_last - G)
#pragma unroll
      for (int t = 0; t < NKT; ++t) {
        if (chan) {
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) S[t][jj] *= svec[R::vDecC + 16 * t + 4 * g + jj];
        } else if (headdecay) {
          S[t] *= svec[R::vMisc];
        }
      }
      if (headdecay || rawk) {
        // the per-token factor goes on D's rows
#pragma unroll
        for (int st = 0; st < NB; ++st) {
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) Dl[st][jj] *= svec[R::vEF + 16 * st + 4 * g + jj];
        }
      }
      if constexpr (rawk) {
        // D in two bf16 parts (hi + lo), k as it is
        bf16x8 Db[NH];
        bf16x8 Dlo[NH];
#pragma unroll
        for (int m = 0; m < NH; ++m) {
          const f32x4 d1 = 2 * m + 1 < NB ? Dl[2 * m + 1] : f32x4{0, 0, 0, 0};
          Db[m] = bf_from_acc(Dl[2 * m], d1);
          Dlo[m] = bf_lo(Dl[2 * m], d1, Db[m]);
        }
#pragma unroll
        for (int t = 0; t < NKT; ++t) {
#pragma unroll
          for (int m = 0; m < NH; ++m) {
            const bf16x8 kt = __builtin_bit_cast(bf16x8, fr.tok(sK, m, t, 2 * m + 1 < NB));
            mma_bf(S[t], kt, Db[m]);
            mma_bf(S[t], kt, Dlo[m]);
          }
        }
      } else {
        if (headdecay) {
#pragma unroll
          for (int m = 0; m < NH; ++m)
            Df[m] = M::from_acc(Dl[2 * m], 2 * m + 1 < NB ? Dl[2 * m + 1] : f32x4{0, 0, 0, 0});
        }
        const unsigned char* KY = chan ? sKF : sK;
#pragma unroll
        for (int t = 0; t < NKT; ++t) {
#pragma unroll
          for (int m = 0; m < NH; ++m)
            M::mma(S[t], fr.tok(KY, m, t, 2 * m + 1 < NB), Df[m]);
        }
      }
      if constexpr (rawk) form_out();
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) Oprev[rt] = Ol[rt];
      if constexpr (rawk) store_out(c);
    } else {
      // helper: the next chunk's copies; with raw rows its share of this
      // chunk's P between the q, k rows and the rest
      if (pre) issue(c + 1, smem + (cur ^ 1) * L::kBuf, std::integral_constant<int, hp ? 1 : 0>{});
      if constexpr (hp) {
        const unsigned char* bq = smem + cur * L::kBuf;
        const unsigned char* sQ = bq + R::oQ;
        const unsigned char* sK = bq + R::oK;
        const float* svec = reinterpret_cast<const float*>(bq + R::oVec);
        // Block (ib, jb) of P: P_ij = fq_i fk_j exp(G_i - G_j) q_i . k_j for
        // j <= i, else 0 (the raw products come transposed: tokens j by
        // tokens i), the fp16 half jb & 1 of operand fragment pf_n(ib, jb / 2).
        // q's row factor comes from the q fragments (a lane's 8 channels per
        // k step; the 4 lane groups of a row hold its other channels); the
        // helper with block (ib, 0) also puts it in FQ.  The blocks of a helper
        // are fixed at compile time (one code path per helper).
        auto share = [&](auto hh_) {
          constexpr int hh = decltype(hh_)::value;
          auto mine = [](int b) { return b * NHELP / NBLK == hh; };
          // every operand first (loads are not moved past the fragment
          // stores below), then the products, then the stores
          bf16x8 qf[NB][NKP], kf[NB][NKP];
          float fq[NB], gi[NB];
          f32x4 fk[NB], gj[NB], acc[NBLK];
          static_for<NB>([&](auto r_) {
            constexpr int r = decltype(r_)::value;
            constexpr bool row = [] { for (int b = 0; b < NBLK; ++b) if (b * NHELP / NBLK == hh && blk_ib(b, NB) == r) return true; return false; }();
            constexpr bool col = [] { for (int b = 0; b < NBLK; ++b) if (b * NHELP / NBLK == hh && blk_jb(b, NB) == r) return true; return false; }();
            if constexpr (row) {
#pragma unroll
              for (int m = 0; m < NKP; ++m) qf[r][m] = __builtin_bit_cast(bf16x8, fr.kq(sQ, r, m));
              gi[r] = headdecay ? svec[R::vG + 16 * r + l16] : 0.f;
            }
            if constexpr (col) {
#pragma unroll
              for (int m = 0; m < NKP; ++m) kf[r][m] = __builtin_bit_cast(bf16x8, fr.kq(sK, r, m));
              fk[r] = *reinterpret_cast<const f32x4*>(svec + R::vFK + 16 * r + 4 * g);
              gj[r] = headdecay ? *reinterpret_cast<const f32x4*>(svec + R::vG + 16 * r + 4 * g) : f32x4{0, 0, 0, 0};
            }
          });
          static_for<NBLK>([&](auto b_) {
            constexpr int b = decltype(b_)::value, ib = blk_ib(b, NB), jb = blk_jb(b, NB);
            if constexpr (mine(b)) {
              acc[b] = f32x4{0, 0, 0, 0};
#pragma unroll
              for (int m = 0; m < NKP; ++m) mma_bf(acc[b], kf[jb][m], qf[ib][m]);
            }
          });
          static_for<NB>([&](auto r_) {
            constexpr int r = decltype(r_)::value;
            constexpr bool row = [] { for (int b = 0; b < NBLK; ++b) if (b * NHELP / NBLK == hh && blk_ib(b, NB) == r) return true; return false; }();
            if constexpr (row) {
              float s0 = 0.f, s1 = 0.f;   // two chains of dependent dot products
#pragma unroll
              for (int m = 0; m < NKP; m += 2) {
                s0 = sumsq_bf(qf[r][m], s0);
                if (m + 1 < NKP) s1 = sumsq_bf(qf[r][m + 1], s1);
              }
              fq[r] = p.scale * (p.l2norm ? inv_norm(xor32_sum(xor16_sum(s0 + s1))) : 1.f);
              // the helper with the row's first block publishes its factor
              constexpr bool pub = [] { for (int b = 0; b < NBLK; ++b) if (b * NHELP / NBLK == hh && blk_ib(b, NB) == r && blk_jb(b, NB) == 0) return true; return false; }();
              if (pub && g == 0) sfq[16 * r + l16] = fq[r];
            }
          });
          static_for<NBLK>([&](auto b_) {
            constexpr int b = decltype(b_)::value, ib = blk_ib(b, NB), jb = blk_jb(b, NB);
            if constexpr (mine(b)) {
              f16x4 hv;
#pragma unroll
              for (int jj = 0; jj < 4; ++jj) {
                float x = acc[b][jj] * fq[ib] * fk[jb][jj];
                if (headdecay) x *= __expf(gi[ib] - gj[jb][jj]);
                hv[jj] = static_cast<_Float16>((jb < ib || 4 * g + jj <= l16) ? x : 0.f);
              }
              *reinterpret_cast<f16x4*>(smem + L::oPF + pf_n(ib, jb / 2) * 1024 + lane * 16 + (jb & 1) * 8) = hv;
            }
          });
        };
        static_for<NHELP>([&](auto hh_) {
          if (hw == decltype(hh_)::value) share(hh_);
        });
        if (lane == 0) __hip_atomic_store(&pflags[hw], c + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        if (pre) issue(c + 1, smem + (cur ^ 1) * L::kBuf, std::integral_constant<int, 2>{});
      }
    }
    if (c + 1 < nchunks) {
      if (L::NBUF == 1) {
        lds_barrier();              // every wave is done with the only buffer
        if constexpr (!own) issue(c + 1, smem, std::integral_constant<int, 0>{});
      }
      // (only the helpers wait: the owners' own memory operations are the
      // output stores, which nothing here reads)
      if constexpr (!own) finish(c + 1, L::NBUF == 2 ? smem + (cur ^ 1) * L::kBuf : smem);
      lds_barrier();                // the next chunk is visible to all waves
    }
  };

  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, L::NBUF == 2 ? 1 : 0>;
  if (owner) {
    for (int c = 0; c < nchunks; c += 2) {
      step(C0{}, std::true_type{}, c);
      if (c + 1 < nchunks) step(C1{}, std::true_type{}, c + 1);
    }
  } else {
    for (int c = 0; c < nchunks; c += 2) {
      step(C0{}, std::false_type{}, c);
      if (c + 1 < nchunks) step(C1{}, std::false_type{}, c + 1);
    }
  }

  // no load may still be landing in LDS when the workgroup ends
  if (!owner) wait_vm();
  if constexpr (!rawk) {
    if (owner && nchunks > 0) store_out(nchunks - 1);
  }
  if (owner) {
#pragma unroll
    for (int t = 0; t < NKT; ++t) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        p.state[sidx(srow(t, j))] = S[t][j];
    }
  }
}

// ---------------------------------------------------------------- launcher --

inline hipError_t set_max_lds(const void* fn) {
  return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(kMaxLds));
}

template <int DK, int DVS, int C, typename In, int DECAY>
hipError_t launch_two(const PrepParams& pp, int nwg_prep, const StateParams& sp, int nwg_state,
                      hipStream_t s) {
  using OpT = typename OpOf<In>::T;
  constexpr bool chan = DECAY == DECAY_CHANNEL;
  using LP = PrepLayout<DK, C, sizeof(OpT), RecLayout<DK, C, sizeof(OpT), chan>::kRawK>;
  using LS = StateLayout<DK, DVS, C, sizeof(OpT), sizeof(In), chan>;
  if constexpr (LP::bytes(chan) > kMaxLds || LS::bytes > kMaxLds) {
    return hipErrorInvalidConfiguration;   // never instantiated as kernels
  } else {
    auto fp0 = prep_kernel<DK, C, In, DECAY, false>;
    auto fp1 = prep_kernel<DK, C, In, DECAY, true>;
    auto fs = state_kernel<DK, DVS, C, In, DECAY>;
    const auto fp = (pp.tf.A_log || pp.tf.beta_mode) ? fp1 : fp0;
    static bool attr_set = false;   // per instantiation; benign race: the calls are idempotent
    hipError_t e = hipSuccess;
    if (!attr_set) {
      e = set_max_lds(reinterpret_cast<const void*>(fp0));
      if (e != hipSuccess) return e;
      e = set_max_lds(reinterpret_cast<const void*>(fp1));
      if (e != hipSuccess) return e;
      e = set_max_lds(reinterpret_cast<const void*>(fs));
      if (e != hipSuccess) return e;
      attr_set = true;
    }
    fp<<<dim3(nwg_prep), dim3(kPrepThreads), LP::bytes(chan), s>>>(pp);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    fs<<<dim3(nwg_state), dim3(64 * state_waves<DVS>()), LS::bytes, s>>>(sp);
    return hipGetLastError();
  }
}

// Shape tables shared by the host planning and the dispatch.
#define KDA_FOR_SHAPES(X)                                                                \
  X(32, 16, 16) X(32, 32, 16) X(32, 64, 16) X(64, 16, 16) X(64, 32, 16) X(64, 64, 16)    \
  X(128, 16, 16) X(128, 32, 16) X(128, 64, 16)                                           \
  X(32, 16, 32) X(32, 32, 32) X(32, 64, 32) X(64, 16, 32) X(64, 32, 32) X(64, 64, 32)    \
  X(128, 16, 32) X(128, 32, 32) X(128, 64, 32)                                           \
  X(32, 16, 64) X(32, 32, 64) X(32, 64, 64) X(64, 16, 64) X(64, 32, 64) X(64, 64, 64)    \
  X(128, 16, 64) X(128, 32, 64) X(128, 64, 64)

// LDS bytes of the larger of the two kernels, 0 for an unknown shape.
template <int OpBytes, int ActBytes>
size_t lds_bytes(int DK, int DVS, int C, bool chan) {
#define KDA_L(dk, dvs, c)                                                                  \
  if (DK == dk && DVS == dvs && C == c) {                                                  \
    const size_t a = chan ? PrepLayout<dk, c, OpBytes, false>::bytes(true)                 \
                          : PrepLayout<dk, c, OpBytes, RecLayout<dk, c, OpBytes, false>::kRawK>::bytes(false); \
    const size_t b = chan ? StateLayout<dk, dvs, c, OpBytes, ActBytes, true>::bytes        \
                          : StateLayout<dk, dvs, c, OpBytes, ActBytes, false>::bytes;      \
    return a > b ? a : b;                                                                  \
  }
  KDA_FOR_SHAPES(KDA_L)
#undef KDA_L
  return 0;
}

// Workspace bytes of one chunk's record.
template <int OpBytes>
size_t record_bytes(int DK, int C, bool chan) {
#define KDA_R(dk, c)                                                                       \
  if (DK == dk && C == c)                                                                  \
    return chan ? RecLayout<dk, c, OpBytes, true>::gBytes : RecLayout<dk, c, OpBytes, false>::gBytes;
  KDA_R(32, 16) KDA_R(64, 16) KDA_R(128, 16) KDA_R(32, 32) KDA_R(64, 32) KDA_R(128, 32)
  KDA_R(32, 64) KDA_R(64, 64) KDA_R(128, 64)
#undef KDA_R
  return 0;
}

template <typename In, int DECAY>
hipError_t launch_any(int DK, int DVS, int C, const PrepParams& pp, int nwg_prep,
                      const StateParams& sp, int nwg_state, hipStream_t s) {
#define KDA_C(dk, dvs, c)                                                                  \
  if (DK == dk && DVS == dvs && C == c)                                                    \
    return launch_two<dk, dvs, c, In, DECAY>(pp, nwg_prep, sp, nwg_state, s);
  KDA_FOR_SHAPES(KDA_C)
#undef KDA_C
  return hipErrorInvalidValue;
}

// One instantiation unit per (activation dtype, decay kind): chunked_<dtype>_d<kind>.hip.
#define KDA_DECLARE_LAUNCH(name)                                                           \
  hipError_t name(int DK, int DVS, int C, const PrepParams& pp, int nwg_prep,              \
                  const StateParams& sp, int nwg_state, hipStream_t s);
KDA_DECLARE_LAUNCH(launch_bf16_d0)
KDA_DECLARE_LAUNCH(launch_bf16_d1)
KDA_DECLARE_LAUNCH(launch_bf16_d2)
KDA_DECLARE_LAUNCH(launch_f32_d0)
KDA_DECLARE_LAUNCH(launch_f32_d1)
KDA_DECLARE_LAUNCH(launch_f32_d2)
#undef KDA_DECLARE_LAUNCH

}  // namespace chunked
}  // namespace kda
