/*
 * kda.h -- C ABI of the MI355X (gfx950) gated delta-rule forward library.
 *
 * The operation (ejkernel "kernel_delta_attention._interface", section "Kernel
 * Delta Attention", the core recurrence and its parameter list): per
 * (batch, head) a [DK, DV] fp32 state S (rows = key channels) evolves as
 *
 *     S_t = diag(exp(decay_t)) S_{t-1} + k_t (beta_t (v_t - S_{t-1}^T k_t))^T
 *     o_t = S_t^T q_t
 *
 * where q_t and k_t are first divided by their L2 norm (if use_qk_l2norm) and
 * q_t is multiplied by softmax_scale.  The delta term reads the previous state
 * before it is decayed, as the recurrence is printed.  decay is log-space and
 * is either absent, one value per (token, head) (the scalar gate of TileOPs
 * GDNFwdOp), or one value per (token, head, key channel) (the per-key-channel
 * gate of TileOPs KDAFwdOp, which scales the state rows).  beta is used as
 * given (TileOPs DeltaNetFwdOp: already transformed) unless the transform
 * flags below ask for the raw-gate / raw-beta inputs of GDNFwdOp and KDAFwdOp.
 *
 * Conventions common to every entry point:
 *
 *  - Every tensor pointer is a DEVICE pointer, owned by the caller, dense and
 *    row-major in the shape stated.  The library never allocates, frees or
 *    keeps device memory: the chunked entry points take a caller-owned
 *    device workspace (size query below).  Calls keep no state between them
 *    and need no init; they are thread-safe as long as concurrent calls do
 *    not share a workspace or an output.
 *  - Activations (q, k, v, beta, decay) share one dtype, KDA_F32 or KDA_BF16.
 *    Outputs o are fp32; states are fp32 (TileOPs DeltaNetFwdOp: the
 *    recurrent state is FP32 and belongs to the caller).
 *  - softmax_scale <= 0 or NaN means the default DK^-0.5 (ejkernel kda:
 *    no scale given means the inverse square root of the head size; TileOPs
 *    GLA ops: non-positive means the default).  use_qk_l2norm != 0 normalises q and k by max(||x||_2, 1e-12).
 *  - decay must be <= 0 (ejkernel kda parameter list: the decay is non-positive); the
 *    kernels rely on it to keep decay factors <= 1 and do not check it.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *    the call returns without synchronising.  The return value reports
 *    argument validation (nothing is launched when it fails) and launch
 *    errors; a device-side fault surfaces at the caller's next
 *    synchronisation.
 *  - Heads (TileOPs GDNFwdOp / KDAFwdOp): q and k have H heads; v, beta,
 *    decay, o and the states have HV recurrent heads, a multiple of H, and
 *    value head hv reads q/k head hv / (HV / H) (consecutive value heads
 *    share a q/k head).  HV == H is the plain case.
 *  - State layout: key-major [.., HV, DK, DV] (state_v_first = 0) or
 *    value-major [.., HV, DV, DK] (state_v_first = 1, TileOPs state_v_first);
 *    initial and final states use the same layout.  Other values:
 *    KDA_ERR_VALUE.
 *  - Supported sizes: DK, DV in {32, 64, 128}; B, H >= 1; 1 <= HV <= 65535
 *    with HV % H == 0; T >= 0 with B*T*HV*max(DK,DV) < 2^31.
 *  - Input transforms, the trailing (A_log, dt_bias, lower_bound, transforms)
 *    of every entry point (TileOPs "Linear Attention Operators", GDNFwdOp and
 *    KDAFwdOp: use_gate_in_kernel, lower_bound, use_beta_sigmoid_in_kernel,
 *    allow_neg_eigval; the gate formula is ejkernel's kda_decay).
 *    `transforms` is a bit set of kda_transform; 0 takes decay and beta as
 *    given, and then A_log, dt_bias and lower_bound are not read.
 *      KDA_TF_GATE: decay holds the raw gate; the kernels use
 *        decay = -exp(A_log[h]) * softplus(gate + dt_bias)
 *        with A_log DEVICE fp32 [HV] (required) and dt_bias DEVICE fp32 [HV]
 *        for KDA_DECAY_HEAD or [HV, DK] for KDA_DECAY_CHANNEL (NULL = 0).
 *        The result is <= 0 by construction.
 *      KDA_TF_LOWER_BOUND (with KDA_TF_GATE): decay = max(decay, lower_bound),
 *        a floor of the forget gate in log space; lower_bound must be <= 0.
 *      KDA_TF_BETA_SIGMOID: beta holds logits; beta = sigmoid(beta).
 *      KDA_TF_NEG_EIGVAL (with KDA_TF_BETA_SIGMOID): beta = 2 sigmoid(beta).
 *    The transforms are computed in fp32 inside the kernels that read decay
 *    and beta; no transformed copy is written.  KDA_ERR_VALUE for unknown
 *    bits, a flag without the one it needs, KDA_TF_GATE with
 *    KDA_DECAY_NONE, or lower_bound > 0 or NaN; KDA_ERR_NULL for
 *    KDA_TF_GATE with A_log NULL (T > 0).
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KDA_OK = 0,
  KDA_ERR_NULL = 1,        /* a required pointer is NULL                     */
  KDA_ERR_SHAPE = 2,       /* a size is out of range or inconsistent         */
  KDA_ERR_UNSUPPORTED = 3, /* DK/DV/chunk/dtype/decay kind not implemented   */
  KDA_ERR_VALUE = 4,       /* invalid transform flags, floor or state layout */
  KDA_ERR_HIP = 5,         /* the HIP runtime reported an error at launch    */
  KDA_ERR_WORKSPACE = 6    /* workspace NULL, misaligned or too small        */
} kda_status;

typedef enum { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype;

typedef enum {
  KDA_TF_GATE = 1,          /* decay is the raw gate (needs A_log)          */
  KDA_TF_LOWER_BOUND = 2,   /* floor the computed decay at lower_bound      */
  KDA_TF_BETA_SIGMOID = 4,  /* beta is a logit: sigmoid(beta)               */
  KDA_TF_NEG_EIGVAL = 8     /* with BETA_SIGMOID: 2 sigmoid(beta)           */
} kda_transform;

typedef enum {
  KDA_DECAY_NONE = 0,    /* decay ignored (may be NULL): no decay             */
  KDA_DECAY_HEAD = 1,    /* decay [.., HV]: one log-space value per token-head */
  KDA_DECAY_CHANNEL = 2  /* decay [.., HV, DK]: one per token-head-key channel */
} kda_decay_kind;

/*
 * Chunked forward: "parallel within chunks, sequential across chunks"
 * (ejkernel kda, section "Algorithm Modes", Chunked), in the WY form of the
 * TileOPs DeltaNet pipeline (prepare_wy_repr, then the forward).
 *
 *   q, k           [B, T, H, DK]  activation dtype
 *   v              [B, T, HV, DV] activation dtype
 *   beta           [B, T, HV]     activation dtype
 *   decay          NULL | [B, T, HV] | [B, T, HV, DK] per decay_kind
 *   initial_state  NULL (zeros) | [B, HV, DK, DV] fp32 ([B, HV, DV, DK]
 *                  value-major)
 *   o              [B, T, HV, DV] fp32, written
 *   final_state    like initial_state, written; may alias initial_state
 *   chunk_size     16, 32 or 64 (ejkernel default 64); the result does not
 *                  depend on it beyond rounding.  T need not be a multiple.
 *
 * Two kernels run on `stream`: a chunk-parallel one that prepares every
 * chunk (normalisation, gate sums, the WY inverse, decayed operands) and a
 * sequential one that carries the state through the chunks and writes o.
 * The prepared chunks pass through `workspace`, DEVICE memory owned by the
 * caller, 16-byte aligned, of `workspace_bytes` bytes; its contents on entry
 * do not matter and are garbage on return.  kda_fwd_chunked_workspace_bytes
 * gives the size that lets one launch pair cover the whole sequence.  A
 * smaller workspace works too, down to the size that query gives for
 * T = chunk_size (one chunk of every head): the chunks are then processed in
 * segments, each launch pair handing its final state to the next (the same
 * result, bitwise).  The workspace must not be used by anything else until
 * the call's work on `stream` has finished.
 *
 * T == 0 copies initial_state (or zeros) to final_state; then q, k, v, beta,
 * decay and o are not read and may be NULL.
 * Errors: KDA_ERR_NULL if final_state is NULL, or (T > 0) q/k/v/beta/o is
 * NULL or decay is NULL with decay_kind != NONE; KDA_ERR_SHAPE for negative or overflowing sizes;
 * KDA_ERR_UNSUPPORTED for other DK/DV/chunk/dtype/decay_kind values;
 * KDA_ERR_WORKSPACE (T > 0) if workspace is NULL, not 16-byte aligned or
 * smaller than one chunk of every head; KDA_ERR_HIP if a launch fails.
 */
int kda_fwd_chunked(const void* q, const void* k, const void* v, const void* beta,
                    const void* decay, int decay_kind, const float* initial_state,
                    float* o, float* final_state,
                    int B, int T, int H, int HV, int DK, int DV, int dtype,
                    float softmax_scale, int use_qk_l2norm, int state_v_first, int chunk_size,
                    const float* A_log, const float* dt_bias, float lower_bound,
                    int transforms, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Workspace bytes for kda_fwd_chunked with these sizes and types to run the
 * whole sequence in one launch pair: one record per (batch, value head,
 * chunk).  A host-only query; 0 when T == 0 (no workspace is read) or when
 * the arguments are invalid or unsupported (the call itself reports which).
 * Called with T = chunk_size it gives the least workspace the call accepts.
 */
size_t kda_fwd_chunked_workspace_bytes(int B, int T, int H, int HV, int DK, int DV, int dtype,
                                       int decay_kind, int chunk_size);

/*
 * Chunked forward over packed variable-length sequences (TileOPs
 * DeltaNetFwdOp / GDNFwdOp / KDAFwdOp: passing cu_seqlens selects the packed
 * varlen mode, the token tensors have B == 1 and N is the number of packed
 * sequences).  Same computation as kda_fwd_chunked for each sequence on its
 * own; chunks never cross a sequence end.
 *
 *   q, k           [1, T, H, DK]  the N sequences back to back
 *   v              [1, T, HV, DV]
 *   beta           [1, T, HV]
 *   decay          NULL | [1, T, HV] | [1, T, HV, DK] per decay_kind
 *   cu_seqlens     DEVICE int32 [N + 1]: sequence n is tokens
 *                  [cu_seqlens[n], cu_seqlens[n + 1])
 *   cu_seqlens_host HOST int32 [N + 1], the same values (sizes the launch)
 *   initial_state  NULL (zeros) | [N, HV, DK, DV] fp32 ([N, HV, DV, DK]
 *                  value-major)
 *   o              [1, T, HV, DV] fp32, written
 *   final_state    like initial_state, written; may alias initial_state
 *
 * An empty sequence passes its initial state through.  The caller-owned
 * workspace (as for kda_fwd_chunked) holds the records of all chunks of all
 * sequences at once and the sequences' chunk offsets: at least
 * kda_fwd_chunked_varlen_workspace_bytes for the same offsets (no
 * segmentation).
 * Errors as kda_fwd_chunked, plus: KDA_ERR_NULL if cu_seqlens or
 * cu_seqlens_host is NULL; KDA_ERR_SHAPE if N < 1, cu_seqlens_host[0] != 0,
 * cu_seqlens_host[N] != T or the offsets decrease; KDA_ERR_WORKSPACE (T > 0)
 * if workspace is NULL, misaligned or smaller than that size.
 */
int kda_fwd_chunked_varlen(const void* q, const void* k, const void* v, const void* beta,
                           const void* decay, int decay_kind, const float* initial_state,
                           float* o, float* final_state, const int* cu_seqlens,
                           const int* cu_seqlens_host, int N,
                           int T, int H, int HV, int DK, int DV, int dtype,
                           float softmax_scale, int use_qk_l2norm, int state_v_first,
                           int chunk_size,
                           const float* A_log, const float* dt_bias, float lower_bound,
                           int transforms, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * Workspace bytes kda_fwd_chunked_varlen needs for the N + 1 HOST offsets
 * cu_seqlens_host (the records of every chunk of every sequence and head, and
 * the chunk offsets).  0 when the sequences hold no token, or when the
 * arguments are invalid or unsupported (the call itself reports which).
 */
size_t kda_fwd_chunked_varlen_workspace_bytes(const int* cu_seqlens_host, int N, int H, int HV,
                                              int DK, int DV, int dtype, int decay_kind,
                                              int chunk_size);
/*
 * Recurrent forward: the pure sequential scan (ejkernel kda, section
 * "Algorithm Modes", Recurrent).  Same arguments and errors as
 * kda_fwd_chunked without chunk_size and the workspace.  Computes in fp32
 * throughout.
 */
int kda_fwd_recurrent(const void* q, const void* k, const void* v, const void* beta,
                      const void* decay, int decay_kind, const float* initial_state,
                      float* o, float* final_state,
                      int B, int T, int H, int HV, int DK, int DV, int dtype,
                      float softmax_scale, int use_qk_l2norm, int state_v_first,
                      const float* A_log, const float* dt_bias, float lower_bound,
                      int transforms, void* stream);

/*
 * Single-step decode (ejkernel kda, the single-step mode for one
 * token with an initial state; the closed form of TileOPs
 * DeltaNetRecurrentFwdOp extended with the gate): one token for every
 * (batch, head), the state updated IN PLACE.
 *
 *   q, k   [B, H, DK]; v [B, HV, DV]; beta [B, HV] (activation dtype)
 *   decay  NULL | [B, HV] | [B, HV, DK] per decay_kind
 *   state  [B, HV, DK, DV] fp32 ([B, HV, DV, DK] value-major), read then
 *          overwritten with the new state
 *   o      [B, HV, DV] fp32, written (must not overlap state)
 *
 * Errors as kda_fwd_chunked (state must be non-NULL).
 */
int kda_decode_step(const void* q, const void* k, const void* v, const void* beta,
                    const void* decay, int decay_kind, float* state, float* o,
                    int B, int H, int HV, int DK, int DV, int dtype,
                    float softmax_scale, int use_qk_l2norm, int state_v_first,
                    const float* A_log, const float* dt_bias, float lower_bound,
                    int transforms, void* stream);

/*
 * Allocation-free chunked forward, for callers that cannot allocate device
 * memory (code under HIP graph capture, serving loops and harnesses that
 * forbid allocation): kda_fwd_chunked with the same arguments, minus the
 * workspace.  The per-chunk records go to a fixed scratch array of
 * KDA_NOALLOC_WORKSPACE_BYTES that the library holds on each device it runs
 * on (its own copy per device, kept until the process ends).  Sequences
 * longer than the scratch holds are processed in segments of chunks, as
 * kda_fwd_chunked does with a small workspace (bitwise the same result).
 * The call allocates and frees nothing, and needs nothing zeroed.
 *
 * Every call on one device shares that device's scratch: calls that overlap
 * on one device (different streams or threads, with no ordering between
 * their work) race and give wrong results.  Calls in one stream are ordered.
 *
 * Errors as kda_fwd_chunked; KDA_ERR_WORKSPACE (T > 0) if one chunk of every
 * head (kda_fwd_chunked_workspace_bytes with T = chunk_size) exceeds
 * KDA_NOALLOC_WORKSPACE_BYTES.
 */
#define KDA_NOALLOC_WORKSPACE_BYTES (64u << 20)
int kda_fwd_chunked_noalloc(const void* q, const void* k, const void* v, const void* beta,
                            const void* decay, int decay_kind, const float* initial_state,
                            float* o, float* final_state,
                            int B, int T, int H, int HV, int DK, int DV, int dtype,
                            float softmax_scale, int use_qk_l2norm, int state_v_first,
                            int chunk_size, const float* A_log, const float* dt_bias,
                            float lower_bound, int transforms, void* stream);

/*
 * Backward: the gradients of a forward call's (o, final_state) with respect
 * to q, k, v, beta, decay and initial_state, given the gradient of o and of
 * the final state (TileOPs "Linear Attention Operators": DeltaNetChunkBwdOp
 * returns dq, dk, dv, dbeta, GLAChunkBwdOp takes do and the final-state
 * gradient; kda-neuron-kernels README, kda_chunk_step_exact_bwd: dq, dk, dv,
 * dg, dbeta, dstate_in).  The forward it differentiates is kda_fwd_chunked /
 * kda_fwd_recurrent with the same inputs and arguments.
 *
 *   q, k, v, beta, decay, initial_state, H, HV, state_v_first, the scale, the
 *                  L2 norm and the transform arguments: as the forward
 *                  (initial_state NULL = zeros)
 *   d_o            [B, T, HV, DV] fp32, the gradient of o
 *   d_final_state  NULL (zeros) | like initial_state, fp32
 *   dq, dk         [B, T, H, DK] fp32, written (the gradients of the raw q,
 *                  k: through the L2 norm and the scale; value heads of a
 *                  group add up)
 *   dv             [B, T, HV, DV] fp32, written
 *   dbeta          [B, T, HV] fp32, written: the gradient of beta as passed
 *                  (of the logits with KDA_TF_BETA_SIGMOID)
 *   ddecay         like decay, fp32, written (ignored with KDA_DECAY_NONE):
 *                  the gradient of decay as passed (of the raw gate with
 *                  KDA_TF_GATE; zero where the floor is taken)
 *   dA_log         with KDA_TF_GATE: [HV] fp32, written
 *   ddt_bias       with KDA_TF_GATE and a dt_bias: like dt_bias, fp32, written
 *   d_initial_state NULL (not written) | like initial_state, fp32, written
 *   workspace      DEVICE, 16-byte aligned, at least kda_bwd_workspace_bytes
 *                  (the state and its gradient at every chunk start, the
 *                  chunks' T and P, per-token factors and, for any decay, a
 *                  per-channel cumulative decay)
 *
 * The backward runs chunk by chunk in the WY form, for every decay kind
 * (chunks of 32 tokens: the states at chunk boundaries forward, their
 * gradients in reverse, then every chunk's local gradients in parallel).
 * All arithmetic is fp32; sums over the value heads of a group (and, for
 * dA_log and ddt_bias, over tokens) are gathered with atomic adds, so those
 * results may differ in the last bits from run to run.
 * Errors as kda_fwd_chunked; KDA_ERR_NULL if (T > 0) d_o, dq, dk, dv, dbeta,
 * (with a decay) ddecay, or (with KDA_TF_GATE) dA_log or (with a dt_bias)
 * ddt_bias is NULL; KDA_ERR_WORKSPACE as for the forward.  T == 0 copies
 * d_final_state (or zeros) to d_initial_state and zeroes dA_log, ddt_bias.
 */
int kda_bwd(const void* q, const void* k, const void* v, const void* beta, const void* decay,
            int decay_kind, const float* initial_state, const float* d_o,
            const float* d_final_state, float* dq, float* dk, float* dv, float* dbeta,
            float* ddecay, float* d_initial_state, int B, int T, int H, int HV, int DK, int DV,
            int dtype, float softmax_scale, int use_qk_l2norm, int state_v_first,
            const float* A_log, const float* dt_bias, float lower_bound, int transforms,
            float* dA_log, float* ddt_bias, void* workspace, size_t workspace_bytes,
            void* stream);

/* Workspace bytes of kda_bwd (host-only), enough for either form; 0 when
 * T == 0 or the sizes are invalid. */
size_t kda_bwd_workspace_bytes(int B, int T, int HV, int DK, int DV);

/* Static, NUL-terminated description of a status code. */
const char* kda_status_string(int status);

/* Library ABI version (major * 100 + minor). */
int kda_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
