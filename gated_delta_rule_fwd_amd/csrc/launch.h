// Internal interface between the C-ABI front end and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>

#include "common.h"

namespace kda {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* beta;
  const void* decay;
  int decay_kind;
  const float* init;   // NULL = zeros (decode: unused)
  float* o;
  float* state;        // final state (decode: state updated in place)
  int B, T, H, DK, DV;   // H: recurrent (value) heads
  int Hk;              // query/key heads; H is a multiple (value head h reads q, k head h / (H / Hk))
  int vfirst;          // states are value-major [.., H, DV, DK] (else key-major [.., H, DK, DV])
  int dtype;           // 0 f32, 1 bf16
  float scale;         // already resolved (> 0)
  int l2norm;
  int chunk;
  Transforms tf;       // raw gate / raw beta handling (all off: inputs as given)
};

// Backward of the forward above: gradients of (o, final state).
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* beta;
  const void* decay;   // NULL with DECAY_NONE
  int decay_kind;
  const float* init;   // NULL = zeros
  const float* dout;   // [B, T, H, DV]
  const float* dfinal; // NULL = zeros
  float* dq;           // [B, T, Hk, DK]
  float* dk;
  float* dv;           // [B, T, H, DV]
  float* dbeta;        // [B, T, H]
  float* ddecay;       // like decay (unused with DECAY_NONE)
  float* dinit;        // NULL: not written
  float* ckpt;         // workspace: bwd_workspace_bytes
  int B, T, H, Hk, DK, DV, dtype;
  float scale;
  int l2norm;
  int vfirst;          // states value-major
  Transforms tf;       // raw gate / raw beta (all off: inputs as given)
  float* dA_log;       // [H] with the raw gate
  float* ddt_bias;     // like dt_bias (with the raw gate and a bias)
};

// Each launcher assumes the front end has validated the arguments.
hipError_t launch_decode(const FwdArgs& a, hipStream_t s);
hipError_t launch_recurrent(const FwdArgs& a, hipStream_t s);
// ws: the caller's workspace of ws_bytes (at least one chunk index's
// records, 16-byte aligned); fewer bytes than all records: segments of chunks.
hipError_t launch_chunked(const FwdArgs& a, void* ws, size_t ws_bytes, hipStream_t s);
// Packed variable-length input: a.B is unused; nseq sequences at the token
// offsets cu (device) / cu_host (host, the same N + 1 values); ws holds the
// records of every chunk, then the nseq + 1 chunk offsets.
hipError_t launch_chunked_varlen(const FwdArgs& a, const int* cu_dev, const int* cu_host, int nseq,
                                 void* ws, hipStream_t s);
hipError_t launch_state_copy(const float* src, float* dst, long n, hipStream_t s);
hipError_t launch_bwd(const BwdArgs& a, hipStream_t s);
size_t bwd_workspace_bytes(int B, int T, int H, int DK, int DV);
// The chunked kernels of the backward, launched by launch_bwd after it has
// cleared what they add into.
hipError_t launch_bwd_chunked(const BwdArgs& a, hipStream_t s);
size_t bwd_chunked_workspace_bytes(int B, int T, int H, int DK, int DV);
// LDS footprint (bytes) of the larger chunked kernel for this shape, 0 if unsupported.
size_t chunked_lds_bytes(int DK, int DV, int chunk, int dtype, int decay_kind);
// The device address of the current device's fixed scratch of
// KDA_NOALLOC_WORKSPACE_BYTES (looked up once per device).
hipError_t noalloc_scratch(void** ptr);
// Workspace bytes of one chunk's record (one head), 0 if unsupported.
size_t chunked_record_bytes(int DK, int chunk, int dtype, int decay_kind);

}  // namespace kda
