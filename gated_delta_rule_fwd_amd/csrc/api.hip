// C-ABI front end of the gated delta-rule library: argument validation and
// dispatch to the kernel launchers.  Declarations and contracts: include/kda.h.
#include <math.h>
#include <stdint.h>

#include "../../include/kda.h"
#include "common.h"
#include "launch.h"

namespace kda {
namespace {

__global__ void state_copy_kernel(const float* __restrict__ src, float* __restrict__ dst, long n) {
  for (long i = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<long>(gridDim.x) * blockDim.x)
    dst[i] = src ? src[i] : 0.f;
}

bool dim_ok(int d) { return d == 32 || d == 64 || d == 128; }

float resolve_scale(float s, int dk) {
  if (!(s > 0.f) || !isfinite(s)) return 1.0f / sqrtf(static_cast<float>(dk));
  return s;
}

// H: query/key heads, HV: recurrent (value) heads, a multiple of H
int check_common(const void* q, const void* k, const void* v, const void* beta, const void* decay,
                 int decay_kind, int B, int T, int H, int HV, int DK, int DV, int dtype,
                 int state_v_first) {
  // with no tokens there is nothing to read: empty tensors may carry NULL
  if (T != 0 && (!q || !k || !v || !beta)) return KDA_ERR_NULL;
  if (decay_kind != KDA_DECAY_NONE && decay_kind != KDA_DECAY_HEAD && decay_kind != KDA_DECAY_CHANNEL)
    return KDA_ERR_UNSUPPORTED;
  if (T != 0 && decay_kind != KDA_DECAY_NONE && !decay) return KDA_ERR_NULL;
  if (B < 1 || H < 1 || HV < 1 || T < 0 || DK < 1 || DV < 1) return KDA_ERR_SHAPE;
  if (HV % H != 0 || HV > 65535) return KDA_ERR_SHAPE;
  if (state_v_first != 0 && state_v_first != 1) return KDA_ERR_VALUE;
  const long long tokens = static_cast<long long>(B) * T * HV;
  const long long widest = static_cast<long long>(DK > DV ? DK : DV);
  if (tokens * widest >= (1LL << 31)) return KDA_ERR_SHAPE;
  if (static_cast<long long>(B) * HV * DK * DV >= (1LL << 31)) return KDA_ERR_SHAPE;
  if (!dim_ok(DK) || !dim_ok(DV)) return KDA_ERR_UNSUPPORTED;
  if (dtype != KDA_F32 && dtype != KDA_BF16) return KDA_ERR_UNSUPPORTED;
  return KDA_OK;
}

int check_transforms(int decay_kind, int T, const float* A_log, float lower_bound, int tf) {
  if (tf & ~(KDA_TF_GATE | KDA_TF_LOWER_BOUND | KDA_TF_BETA_SIGMOID | KDA_TF_NEG_EIGVAL))
    return KDA_ERR_VALUE;
  if ((tf & KDA_TF_GATE) && decay_kind == KDA_DECAY_NONE) return KDA_ERR_VALUE;
  if ((tf & KDA_TF_LOWER_BOUND) && (!(tf & KDA_TF_GATE) || !(lower_bound <= 0.f)))
    return KDA_ERR_VALUE;
  if ((tf & KDA_TF_NEG_EIGVAL) && !(tf & KDA_TF_BETA_SIGMOID)) return KDA_ERR_VALUE;
  if (T != 0 && (tf & KDA_TF_GATE) && !A_log) return KDA_ERR_NULL;
  return KDA_OK;
}

Transforms make_tf(const float* A_log, const float* dt_bias, float lower_bound, int tf) {
  Transforms t;
  const bool gate = (tf & KDA_TF_GATE) != 0;
  t.A_log = gate ? A_log : nullptr;
  t.dt_bias = gate ? dt_bias : nullptr;
  t.lower = (tf & KDA_TF_LOWER_BOUND) ? lower_bound : -INFINITY;
  t.beta_mode = !(tf & KDA_TF_BETA_SIGMOID) ? 0 : (tf & KDA_TF_NEG_EIGVAL) ? 2 : 1;
  return t;
}

FwdArgs make_args(const void* q, const void* k, const void* v, const void* beta, const void* decay,
                  int decay_kind, const float* init, float* o, float* state, int B, int T, int H,
                  int HV, int DK, int DV, int dtype, float scale, int l2, int vfirst, int chunk,
                  const Transforms& tf) {
  FwdArgs a;
  a.tf = tf;
  a.Hk = H;
  a.vfirst = vfirst;
  a.q = q; a.k = k; a.v = v; a.beta = beta;
  a.decay = decay_kind == KDA_DECAY_NONE ? nullptr : decay;
  a.decay_kind = decay_kind;
  a.init = init; a.o = o; a.state = state;
  a.B = B; a.T = T; a.H = HV; a.DK = DK; a.DV = DV; a.dtype = dtype;
  a.scale = resolve_scale(scale, DK);
  a.l2norm = l2 ? 1 : 0;
  a.chunk = chunk;
  return a;
}

int to_status(hipError_t e) { return e == hipSuccess ? KDA_OK : KDA_ERR_HIP; }

bool chunk_ok(int chunk) { return chunk == 16 || chunk == 32 || chunk == 64; }

// Bytes of the chunked records for `chunks` chunk indices of `heads` value
// heads, 0 for an unsupported shape.
size_t records_bytes(long chunks, long heads, int DK, int DV, int dtype, int decay_kind, int chunk) {
  if (!chunk_ok(chunk) || chunked_lds_bytes(DK, DV, chunk, dtype, decay_kind) == 0) return 0;
  return chunked_record_bytes(DK, chunk, dtype, decay_kind) * static_cast<size_t>(chunks) *
         static_cast<size_t>(heads);
}

bool ws_aligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Chunk offsets after the varlen records, 16-byte aligned.
size_t varlen_offsets_at(size_t recs) { return (recs + 15) & ~static_cast<size_t>(15); }

}  // namespace

hipError_t launch_state_copy(const float* src, float* dst, long n, hipStream_t s) {
  if (n == 0 || src == dst) return hipSuccess;
  long blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  state_copy_kernel<<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s>>>(src, dst, n);
  return hipGetLastError();
}

}  // namespace kda

extern "C" {

int kda_fwd_chunked(const void* q, const void* k, const void* v, const void* beta,
                    const void* decay, int decay_kind, const float* initial_state,
                    float* o, float* final_state,
                    int B, int T, int H, int HV, int DK, int DV, int dtype,
                    float softmax_scale, int use_qk_l2norm, int state_v_first, int chunk_size,
                    const float* A_log, const float* dt_bias, float lower_bound, int transforms,
                    void* workspace, size_t workspace_bytes, void* stream) {
  int st = kda::check_common(q, k, v, beta, decay, decay_kind, B, T, H, HV, DK, DV, dtype,
                             state_v_first);
  if (st == KDA_OK) st = kda::check_transforms(decay_kind, T, A_log, lower_bound, transforms);
  if (st != KDA_OK) return st;
  if (!final_state || (T != 0 && !o)) return KDA_ERR_NULL;
  if (chunk_size != 16 && chunk_size != 32 && chunk_size != 64) return KDA_ERR_UNSUPPORTED;
  if (kda::chunked_lds_bytes(DK, DV, chunk_size, dtype, decay_kind) == 0) return KDA_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (T == 0) {
    return kda::to_status(kda::launch_state_copy(initial_state, final_state,
                                                 static_cast<long>(B) * HV * DK * DV, s));
  }
  // the least workspace: one chunk index of every head
  const size_t least = kda::records_bytes(1, static_cast<long>(B) * HV, DK, DV, dtype, decay_kind,
                                          chunk_size);
  if (!workspace || !kda::ws_aligned(workspace) || workspace_bytes < least) return KDA_ERR_WORKSPACE;
  const kda::FwdArgs a = kda::make_args(q, k, v, beta, decay, decay_kind, initial_state, o,
                                        final_state, B, T, H, HV, DK, DV, dtype, softmax_scale,
                                        use_qk_l2norm, state_v_first, chunk_size,
                                        kda::make_tf(A_log, dt_bias, lower_bound, transforms));
  return kda::to_status(kda::launch_chunked(a, workspace, workspace_bytes, s));
}

int kda_fwd_chunked_varlen(const void* q, const void* k, const void* v, const void* beta,
                           const void* decay, int decay_kind, const float* initial_state,
                           float* o, float* final_state, const int* cu_seqlens,
                           const int* cu_seqlens_host, int N,
                           int T, int H, int HV, int DK, int DV, int dtype,
                           float softmax_scale, int use_qk_l2norm, int state_v_first,
                           int chunk_size,
                           const float* A_log, const float* dt_bias, float lower_bound,
                           int transforms, void* workspace, size_t workspace_bytes,
                           void* stream) {
  int st = kda::check_common(q, k, v, beta, decay, decay_kind, 1, T, H, HV, DK, DV, dtype,
                             state_v_first);
  if (st == KDA_OK) st = kda::check_transforms(decay_kind, T, A_log, lower_bound, transforms);
  if (st != KDA_OK) return st;
  if (!final_state || !cu_seqlens || !cu_seqlens_host || (T != 0 && !o)) return KDA_ERR_NULL;
  if (N < 1 || static_cast<long long>(N) * HV * DK * DV >= (1LL << 31)) return KDA_ERR_SHAPE;
  if (cu_seqlens_host[0] != 0 || cu_seqlens_host[N] != T) return KDA_ERR_SHAPE;
  for (int n = 0; n < N; ++n)
    if (cu_seqlens_host[n + 1] < cu_seqlens_host[n]) return KDA_ERR_SHAPE;
  if (chunk_size != 16 && chunk_size != 32 && chunk_size != 64) return KDA_ERR_UNSUPPORTED;
  if (kda::chunked_lds_bytes(DK, DV, chunk_size, dtype, decay_kind) == 0) return KDA_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (T == 0) {
    return kda::to_status(kda::launch_state_copy(initial_state, final_state,
                                                 static_cast<long>(N) * HV * DK * DV, s));
  }
  if (!workspace || !kda::ws_aligned(workspace) ||
      workspace_bytes < kda_fwd_chunked_varlen_workspace_bytes(cu_seqlens_host, N, H, HV, DK, DV,
                                                               dtype, decay_kind, chunk_size))
    return KDA_ERR_WORKSPACE;
  const kda::FwdArgs a = kda::make_args(q, k, v, beta, decay, decay_kind, initial_state, o,
                                        final_state, 1, T, H, HV, DK, DV, dtype, softmax_scale,
                                        use_qk_l2norm, state_v_first, chunk_size,
                                        kda::make_tf(A_log, dt_bias, lower_bound, transforms));
  return kda::to_status(kda::launch_chunked_varlen(a, cu_seqlens, cu_seqlens_host, N, workspace, s));
}

int kda_fwd_chunked_noalloc(const void* q, const void* k, const void* v, const void* beta,
                            const void* decay, int decay_kind, const float* initial_state,
                            float* o, float* final_state,
                            int B, int T, int H, int HV, int DK, int DV, int dtype,
                            float softmax_scale, int use_qk_l2norm, int state_v_first,
                            int chunk_size, const float* A_log, const float* dt_bias,
                            float lower_bound, int transforms, void* stream) {
  int st = kda::check_common(q, k, v, beta, decay, decay_kind, B, T, H, HV, DK, DV, dtype,
                             state_v_first);
  if (st == KDA_OK) st = kda::check_transforms(decay_kind, T, A_log, lower_bound, transforms);
  if (st != KDA_OK) return st;
  if (!final_state || (T != 0 && !o)) return KDA_ERR_NULL;
  if (!kda::chunk_ok(chunk_size)) return KDA_ERR_UNSUPPORTED;
  if (kda::chunked_lds_bytes(DK, DV, chunk_size, dtype, decay_kind) == 0) return KDA_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (T == 0) {
    return kda::to_status(kda::launch_state_copy(initial_state, final_state,
                                                 static_cast<long>(B) * HV * DK * DV, s));
  }
  // the scratch must hold one chunk index of every head (checked before any HIP call)
  const size_t least = kda::records_bytes(1, static_cast<long>(B) * HV, DK, DV, dtype, decay_kind,
                                          chunk_size);
  if (least > KDA_NOALLOC_WORKSPACE_BYTES) return KDA_ERR_WORKSPACE;
  void* ws = nullptr;
  hipError_t e = kda::noalloc_scratch(&ws);
  if (e != hipSuccess) return KDA_ERR_HIP;
  const kda::FwdArgs a = kda::make_args(q, k, v, beta, decay, decay_kind, initial_state, o,
                                        final_state, B, T, H, HV, DK, DV, dtype, softmax_scale,
                                        use_qk_l2norm, state_v_first, chunk_size,
                                        kda::make_tf(A_log, dt_bias, lower_bound, transforms));
  return kda::to_status(kda::launch_chunked(a, ws, KDA_NOALLOC_WORKSPACE_BYTES, s));
}

size_t kda_fwd_chunked_workspace_bytes(int B, int T, int H, int HV, int DK, int DV, int dtype,
                                       int decay_kind, int chunk_size) {
  if (B < 1 || T < 1 || H < 1 || HV < 1 || HV % H != 0) return 0;
  if (!kda::dim_ok(DK) || !kda::dim_ok(DV) || (dtype != KDA_F32 && dtype != KDA_BF16)) return 0;
  if (decay_kind < KDA_DECAY_NONE || decay_kind > KDA_DECAY_CHANNEL || !kda::chunk_ok(chunk_size)) return 0;
  const long chunks = (static_cast<long>(T) + chunk_size - 1) / chunk_size;
  return kda::records_bytes(chunks, static_cast<long>(B) * HV, DK, DV, dtype, decay_kind, chunk_size);
}

size_t kda_fwd_chunked_varlen_workspace_bytes(const int* cu_seqlens_host, int N, int H, int HV,
                                              int DK, int DV, int dtype, int decay_kind,
                                              int chunk_size) {
  if (!cu_seqlens_host || N < 1 || H < 1 || HV < 1 || HV % H != 0) return 0;
  if (!kda::dim_ok(DK) || !kda::dim_ok(DV) || (dtype != KDA_F32 && dtype != KDA_BF16)) return 0;
  if (decay_kind < KDA_DECAY_NONE || decay_kind > KDA_DECAY_CHANNEL || !kda::chunk_ok(chunk_size)) return 0;
  if (cu_seqlens_host[0] != 0) return 0;
  long chunks = 0;
  for (int n = 0; n < N; ++n) {
    const long len = static_cast<long>(cu_seqlens_host[n + 1]) - cu_seqlens_host[n];
    if (len < 0) return 0;
    chunks += (len + chunk_size - 1) / chunk_size;
  }
  if (chunks == 0) return 0;
  const size_t recs = kda::records_bytes(chunks, HV, DK, DV, dtype, decay_kind, chunk_size);
  if (recs == 0) return 0;
  return kda::varlen_offsets_at(recs) + (static_cast<size_t>(N) + 1) * sizeof(int);
}

int kda_fwd_recurrent(const void* q, const void* k, const void* v, const void* beta,
                      const void* decay, int decay_kind, const float* initial_state,
                      float* o, float* final_state,
                      int B, int T, int H, int HV, int DK, int DV, int dtype,
                      float softmax_scale, int use_qk_l2norm, int state_v_first,
                    const float* A_log, const float* dt_bias, float lower_bound, int transforms,
                    void* stream) {
  int st = kda::check_common(q, k, v, beta, decay, decay_kind, B, T, H, HV, DK, DV, dtype,
                             state_v_first);
  if (st == KDA_OK) st = kda::check_transforms(decay_kind, T, A_log, lower_bound, transforms);
  if (st != KDA_OK) return st;
  if (!final_state || (T != 0 && !o)) return KDA_ERR_NULL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (T == 0) {
    return kda::to_status(kda::launch_state_copy(initial_state, final_state,
                                                 static_cast<long>(B) * HV * DK * DV, s));
  }
  const kda::FwdArgs a = kda::make_args(q, k, v, beta, decay, decay_kind, initial_state, o,
                                        final_state, B, T, H, HV, DK, DV, dtype, softmax_scale,
                                        use_qk_l2norm, state_v_first, 0,
                                        kda::make_tf(A_log, dt_bias, lower_bound, transforms));
  return kda::to_status(kda::launch_recurrent(a, s));
}

int kda_decode_step(const void* q, const void* k, const void* v, const void* beta,
                    const void* decay, int decay_kind, float* state, float* o,
                    int B, int H, int HV, int DK, int DV, int dtype,
                    float softmax_scale, int use_qk_l2norm, int state_v_first,
                    const float* A_log, const float* dt_bias, float lower_bound, int transforms,
                    void* stream) {
  int st = kda::check_common(q, k, v, beta, decay, decay_kind, B, 1, H, HV, DK, DV, dtype,
                             state_v_first);
  if (st == KDA_OK) st = kda::check_transforms(decay_kind, 1, A_log, lower_bound, transforms);
  if (st != KDA_OK) return st;
  if (!state || !o) return KDA_ERR_NULL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const kda::FwdArgs a = kda::make_args(q, k, v, beta, decay, decay_kind, state, o, state, B, 1, H,
                                        HV, DK, DV, dtype, softmax_scale, use_qk_l2norm,
                                        state_v_first, 0,
                                        kda::make_tf(A_log, dt_bias, lower_bound, transforms));
  return kda::to_status(kda::launch_decode(a, s));
}

size_t kda_bwd_workspace_bytes(int B, int T, int HV, int DK, int DV) {
  if (B < 1 || T < 1 || HV < 1 || !kda::dim_ok(DK) || !kda::dim_ok(DV)) return 0;
  return kda::bwd_workspace_bytes(B, T, HV, DK, DV);
}

int kda_bwd(const void* q, const void* k, const void* v, const void* beta, const void* decay,
            int decay_kind, const float* initial_state, const float* d_o,
            const float* d_final_state, float* dq, float* dk, float* dv, float* dbeta,
            float* ddecay, float* d_initial_state, int B, int T, int H, int HV, int DK, int DV,
            int dtype, float softmax_scale, int use_qk_l2norm, int state_v_first,
            const float* A_log, const float* dt_bias, float lower_bound, int transforms,
            float* dA_log, float* ddt_bias, void* workspace, size_t workspace_bytes,
            void* stream) {
  int st = kda::check_common(q, k, v, beta, decay, decay_kind, B, T, H, HV, DK, DV, dtype,
                             state_v_first);
  if (st == KDA_OK) st = kda::check_transforms(decay_kind, T, A_log, lower_bound, transforms);
  if (st != KDA_OK) return st;
  if (T != 0 && (!d_o || !dq || !dk || !dv || !dbeta)) return KDA_ERR_NULL;
  if (T != 0 && decay_kind != KDA_DECAY_NONE && !ddecay) return KDA_ERR_NULL;
  if (T != 0 && (transforms & KDA_TF_GATE) && (!dA_log || (dt_bias && !ddt_bias))) return KDA_ERR_NULL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (T == 0) {
    // no tokens: the initial state's gradient is the final state's (the
    // gradients of A_log and dt_bias are zero)
    hipError_t e = hipSuccess;
    if ((transforms & KDA_TF_GATE) && dA_log) e = kda::launch_state_copy(nullptr, dA_log, HV, s);
    if (e == hipSuccess && (transforms & KDA_TF_GATE) && dt_bias && ddt_bias)
      e = kda::launch_state_copy(nullptr, ddt_bias,
                                 decay_kind == KDA_DECAY_CHANNEL ? static_cast<long>(HV) * DK : HV, s);
    if (e == hipSuccess && d_initial_state)
      e = kda::launch_state_copy(d_final_state, d_initial_state, static_cast<long>(B) * HV * DK * DV, s);
    return kda::to_status(e);
  }
  if (!workspace || !kda::ws_aligned(workspace) ||
      workspace_bytes < kda::bwd_workspace_bytes(B, T, HV, DK, DV))
    return KDA_ERR_WORKSPACE;
  kda::BwdArgs a;
  a.q = q; a.k = k; a.v = v; a.beta = beta;
  a.decay = decay_kind == KDA_DECAY_NONE ? nullptr : decay;
  a.decay_kind = decay_kind;
  a.init = initial_state; a.dout = d_o; a.dfinal = d_final_state;
  a.dq = dq; a.dk = dk; a.dv = dv; a.dbeta = dbeta;
  a.ddecay = decay_kind == KDA_DECAY_NONE ? nullptr : ddecay;
  a.dinit = d_initial_state;
  a.ckpt = static_cast<float*>(workspace);
  a.B = B; a.T = T; a.H = HV; a.Hk = H; a.DK = DK; a.DV = DV; a.dtype = dtype;
  a.scale = kda::resolve_scale(softmax_scale, DK);
  a.l2norm = use_qk_l2norm ? 1 : 0;
  a.vfirst = state_v_first;
  a.tf = kda::make_tf(A_log, dt_bias, lower_bound, transforms);
  a.dA_log = (transforms & KDA_TF_GATE) ? dA_log : nullptr;
  a.ddt_bias = (transforms & KDA_TF_GATE) && dt_bias ? ddt_bias : nullptr;
  return kda::to_status(kda::launch_bwd(a, s));
}

const char* kda_status_string(int status) {
  switch (status) {
    case KDA_OK: return "ok";
    case KDA_ERR_NULL: return "a required pointer is NULL";
    case KDA_ERR_SHAPE: return "a size is out of range or inconsistent";
    case KDA_ERR_UNSUPPORTED: return "unsupported head size, chunk size, dtype or decay kind";
    case KDA_ERR_VALUE: return "invalid transform flags, lower bound or state layout";
    case KDA_ERR_HIP: return "HIP runtime error at launch";
    case KDA_ERR_WORKSPACE: return "workspace NULL, not 16-byte aligned or too small";
  }
  return "unknown status";
}

int kda_abi_version(void) { return 202; }

}  // extern "C"
