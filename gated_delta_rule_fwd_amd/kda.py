"""Python binding of libkda.so: argument marshalling only.

Every function here checks tensor placement, dtype and shape, allocates the
outputs with torch (device memory is all torch is used for), and calls the
C entry point of the same name on torch's current stream.  All arithmetic
runs in the library's HIP kernels; there is no fallback.  Calls are
asynchronous like any torch op on that stream.
"""

from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkda.so")

KDA_F32, KDA_BF16 = 0, 1
DECAY_NONE, DECAY_HEAD, DECAY_CHANNEL = 0, 1, 2
STATUS = {0: "KDA_OK", 1: "KDA_ERR_NULL", 2: "KDA_ERR_SHAPE", 3: "KDA_ERR_UNSUPPORTED",
          4: "KDA_ERR_VALUE", 5: "KDA_ERR_HIP", 6: "KDA_ERR_WORKSPACE"}
TF_GATE, TF_LOWER_BOUND, TF_BETA_SIGMOID, TF_NEG_EIGVAL = 1, 2, 4, 8
# the fixed per-device scratch of kda_fwd_chunked_noalloc (KDA_NOALLOC_WORKSPACE_BYTES)
NOALLOC_WORKSPACE_BYTES = 64 << 20

_lib = None


class KdaError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        msg = lib().kda_status_string(status).decode()
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({msg})")


def lib() -> ctypes.CDLL:
    """Load libkda.so (built by ``gated_delta_rule_fwd_amd.build``); raise if absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m gated_delta_rule_fwd_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        L.kda_fwd_chunked.argtypes = [vp, vp, vp, vp, vp, i, vp, vp, vp,
                                      i, i, i, i, i, i, i, f, i, i, i, vp, vp, f, i, vp, sz, vp]
        L.kda_fwd_chunked.restype = i
        L.kda_fwd_chunked_noalloc.argtypes = [vp, vp, vp, vp, vp, i, vp, vp, vp,
                                              i, i, i, i, i, i, i, f, i, i, i, vp, vp, f, i, vp]
        L.kda_fwd_chunked_noalloc.restype = i
        L.kda_fwd_chunked_workspace_bytes.argtypes = [i, i, i, i, i, i, i, i, i]
        L.kda_fwd_chunked_workspace_bytes.restype = sz
        L.kda_fwd_chunked_varlen.argtypes = [vp, vp, vp, vp, vp, i, vp, vp, vp, vp, vp, i,
                                             i, i, i, i, i, i, f, i, i, i, vp, vp, f, i, vp, sz,
                                             vp]
        L.kda_fwd_chunked_varlen.restype = i
        L.kda_fwd_chunked_varlen_workspace_bytes.argtypes = [vp, i, i, i, i, i, i, i, i]
        L.kda_fwd_chunked_varlen_workspace_bytes.restype = sz
        L.kda_fwd_recurrent.argtypes = [vp, vp, vp, vp, vp, i, vp, vp, vp,
                                        i, i, i, i, i, i, i, f, i, i, vp, vp, f, i, vp]
        L.kda_fwd_recurrent.restype = i
        L.kda_decode_step.argtypes = [vp, vp, vp, vp, vp, i, vp, vp,
                                      i, i, i, i, i, i, f, i, i, vp, vp, f, i, vp]
        L.kda_decode_step.restype = i
        L.kda_bwd.argtypes = [vp, vp, vp, vp, vp, i, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                              i, i, i, i, i, i, i, f, i, i, vp, vp, f, i, vp, vp, vp, sz, vp]
        L.kda_bwd.restype = i
        L.kda_bwd_workspace_bytes.argtypes = [i, i, i, i, i]
        L.kda_bwd_workspace_bytes.restype = sz
        L.kda_status_string.argtypes = [i]
        L.kda_status_string.restype = ctypes.c_char_p
        L.kda_abi_version.argtypes = []
        L.kda_abi_version.restype = i
        _lib = L
    return _lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return KDA_F32
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    raise TypeError(f"activations must be float32 or bfloat16, got {t.dtype}")


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check_act(name, t, shape, dtype, device):
    if t is None:
        raise ValueError(f"{name} is required")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_state(name, t, shape, device):
    if t is None:
        return
    if t.device != device or t.dtype != torch.float32 or tuple(t.shape) != tuple(shape) \
            or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous float32 tensor of shape {tuple(shape)} "
                         f"on {device}")


def _scale(softmax_scale):
    return 0.0 if softmax_scale is None else float(softmax_scale)


def _decay_kind(decay, lead, dk):
    if decay is None:
        return DECAY_NONE
    if tuple(decay.shape) == tuple(lead):
        return DECAY_HEAD
    if tuple(decay.shape) == tuple(lead) + (dk,):
        return DECAY_CHANNEL
    raise ValueError(f"decay has shape {tuple(decay.shape)}; expected {tuple(lead)} or "
                     f"{tuple(lead) + (dk,)}")


def _transforms(kind, H, DK, dev, use_gate_in_kernel, A_log, dt_bias, lower_bound,
                use_beta_sigmoid_in_kernel, allow_neg_eigval):
    """(A_log, dt_bias, lower_bound, flags) for the C entry points.  The
    flag combinations are checked by the library (KDA_ERR_VALUE)."""
    flags = 0
    if use_gate_in_kernel:
        flags |= TF_GATE
        _check_state("A_log", A_log, (H,), dev)
        if A_log is None:
            raise ValueError("use_gate_in_kernel needs A_log [H]")
        _check_state("dt_bias", dt_bias, (H, DK) if kind == DECAY_CHANNEL else (H,), dev)
    else:
        A_log = dt_bias = None
    if lower_bound is not None:
        flags |= TF_LOWER_BOUND
    if use_beta_sigmoid_in_kernel:
        flags |= TF_BETA_SIGMOID
    if allow_neg_eigval:
        flags |= TF_NEG_EIGVAL
    lb = 0.0 if lower_bound is None else float(lower_bound)
    return _ptr(A_log), _ptr(dt_bias), lb, flags


def _workspace(workspace, nbytes, dev):
    """The caller's workspace (a device tensor of at least the bytes the
    library asks for; any dtype, contiguous), or a fresh torch.empty one."""
    if workspace is None:
        return torch.empty(max(nbytes, 1), device=dev, dtype=torch.uint8)
    if workspace.device != dev or not workspace.is_contiguous():
        raise ValueError(f"workspace must be a contiguous tensor on {dev}")
    return workspace


def chunked_workspace_bytes(B, T, H, HV, DK, DV, dtype, decay_kind, chunk_size=64):
    """Bytes of workspace for one launch pair of fwd_chunked over the whole
    sequence (kda_fwd_chunked_workspace_bytes); ``dtype`` a torch dtype or
    the library's code.  With T = chunk_size: the least it accepts."""
    code = dtype if isinstance(dtype, int) else (KDA_F32 if dtype == torch.float32 else KDA_BF16)
    return int(lib().kda_fwd_chunked_workspace_bytes(B, T, H, HV, DK, DV, code, decay_kind,
                                                     chunk_size))


def chunked_varlen_workspace_bytes(cu_seqlens, H, HV, DK, DV, dtype, decay_kind, chunk_size=64):
    """Bytes of workspace fwd_chunked_varlen needs for these offsets
    (kda_fwd_chunked_varlen_workspace_bytes; cu_seqlens N + 1 int offsets)."""
    cu = torch.as_tensor(cu_seqlens).to("cpu", torch.int32).contiguous()
    code = dtype if isinstance(dtype, int) else (KDA_F32 if dtype == torch.float32 else KDA_BF16)
    return int(lib().kda_fwd_chunked_varlen_workspace_bytes(_ptr(cu), cu.numel() - 1, H, HV, DK,
                                                            DV, code, decay_kind, chunk_size))


def _state_shape(N, HV, DK, DV, state_v_first):
    return (N, HV, DV, DK) if state_v_first else (N, HV, DK, DV)


def _prep_fwd(q, k, v, beta, decay, initial_state, state_v_first=False):
    """q, k [B,T,H,DK]; v [B,T,HV,DV] with HV a multiple of H (value head hv
    reads q/k head hv // (HV // H)); beta, decay and o per value head."""
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q must be [B, T, H, DK] and v [B, T, HV, DV]")
    B, T, H, DK = q.shape
    HV, DV = v.shape[2], v.shape[3]
    dev, dt = q.device, q.dtype
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU device")
    _check_act("q", q, (B, T, H, DK), dt, dev)
    _check_act("k", k, (B, T, H, DK), dt, dev)
    _check_act("v", v, (B, T, HV, DV), dt, dev)
    _check_act("beta", beta, (B, T, HV), dt, dev)
    kind = _decay_kind(decay, (B, T, HV), DK)
    if decay is not None:
        _check_act("decay", decay, tuple(decay.shape), dt, dev)
    _check_state("initial_state", initial_state, _state_shape(B, HV, DK, DV, state_v_first), dev)
    return B, T, H, HV, DK, DV, dev, kind


def fwd_chunked(q, k, v, beta, decay=None, initial_state=None, softmax_scale=None,
                use_qk_l2norm=True, chunk_size=64, out=None, final_state=None,
                state_v_first=False, use_gate_in_kernel=False, A_log=None, dt_bias=None,
                lower_bound=None, use_beta_sigmoid_in_kernel=False, allow_neg_eigval=False,
                workspace=None):
    """Chunked forward.  q, k [B,T,H,DK]; v [B,T,HV,DV] (HV a multiple of H);
    beta [B,T,HV]; decay None, [B,T,HV] or [B,T,HV,DK].  Returns (o [B,T,HV,DV]
    fp32, final_state fp32), states [B,HV,DK,DV], or [B,HV,DV,DK] with
    ``state_v_first``.

    Input transforms (all entry points): with ``use_gate_in_kernel`` the
    decay tensor holds the raw gate and the kernels use
    -exp(A_log) * softplus(gate + dt_bias), floored at ``lower_bound`` if
    given (A_log [HV] fp32; dt_bias [HV], or [HV, DK] for a per-channel gate,
    fp32 or None); ``use_beta_sigmoid_in_kernel`` reads beta as logits
    (sigmoid, or 2 * sigmoid with ``allow_neg_eigval``).

    ``workspace``: a device tensor the library may use for the per-chunk
    records (chunked_workspace_bytes gives the size for one launch pair; a
    smaller one, down to one chunk of every head, processes the sequence in
    segments).  None: torch.empty of the full size."""
    B, T, H, HV, DK, DV, dev, kind = _prep_fwd(q, k, v, beta, decay, initial_state, state_v_first)
    tf = _transforms(kind, HV, DK, dev, use_gate_in_kernel, A_log, dt_bias, lower_bound,
                     use_beta_sigmoid_in_kernel, allow_neg_eigval)
    sshape = _state_shape(B, HV, DK, DV, state_v_first)
    o = out if out is not None else torch.empty((B, T, HV, DV), device=dev, dtype=torch.float32)
    _check_state("out", o, (B, T, HV, DV), dev)
    fs = final_state if final_state is not None else torch.empty(sshape, device=dev,
                                                                 dtype=torch.float32)
    _check_state("final_state", fs, sshape, dev)
    need = lib().kda_fwd_chunked_workspace_bytes(B, T, H, HV, DK, DV, _dtype_code(q), kind,
                                                 int(chunk_size))
    ws = _workspace(workspace, need, dev)
    st = lib().kda_fwd_chunked(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(decay), kind,
                               _ptr(initial_state), _ptr(o), _ptr(fs), B, T, H, HV, DK, DV,
                               _dtype_code(q), _scale(softmax_scale), int(bool(use_qk_l2norm)),
                               int(bool(state_v_first)), int(chunk_size), *tf, _ptr(ws),
                               ws.numel() * ws.element_size(), _stream(dev))
    if st != 0:
        raise KdaError("kda_fwd_chunked", st)
    return o, fs


def fwd_chunked_noalloc(q, k, v, beta, decay=None, initial_state=None, softmax_scale=None,
                        use_qk_l2norm=True, chunk_size=64, out=None, final_state=None,
                        state_v_first=False, use_gate_in_kernel=False, A_log=None, dt_bias=None,
                        lower_bound=None, use_beta_sigmoid_in_kernel=False,
                        allow_neg_eigval=False):
    """fwd_chunked through kda_fwd_chunked_noalloc: the library keeps the
    per-chunk records in its fixed per-device scratch, so the C call
    allocates nothing (pass ``out`` and ``final_state`` to allocate nothing
    here either).  Calls that overlap on one device race on that scratch."""
    B, T, H, HV, DK, DV, dev, kind = _prep_fwd(q, k, v, beta, decay, initial_state, state_v_first)
    tf = _transforms(kind, HV, DK, dev, use_gate_in_kernel, A_log, dt_bias, lower_bound,
                     use_beta_sigmoid_in_kernel, allow_neg_eigval)
    sshape = _state_shape(B, HV, DK, DV, state_v_first)
    o = out if out is not None else torch.empty((B, T, HV, DV), device=dev, dtype=torch.float32)
    _check_state("out", o, (B, T, HV, DV), dev)
    fs = final_state if final_state is not None else torch.empty(sshape, device=dev,
                                                                 dtype=torch.float32)
    _check_state("final_state", fs, sshape, dev)
    st = lib().kda_fwd_chunked_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(decay), kind,
                                       _ptr(initial_state), _ptr(o), _ptr(fs), B, T, H, HV, DK,
                                       DV, _dtype_code(q), _scale(softmax_scale),
                                       int(bool(use_qk_l2norm)), int(bool(state_v_first)),
                                       int(chunk_size), *tf, _stream(dev))
    if st != 0:
        raise KdaError("kda_fwd_chunked_noalloc", st)
    return o, fs


def fwd_chunked_varlen(q, k, v, beta, cu_seqlens, decay=None, initial_state=None,
                       softmax_scale=None, use_qk_l2norm=True, chunk_size=64, out=None,
                       final_state=None, state_v_first=False, use_gate_in_kernel=False,
                       A_log=None, dt_bias=None, lower_bound=None,
                       use_beta_sigmoid_in_kernel=False, allow_neg_eigval=False, workspace=None):
    """Chunked forward over N packed sequences (tokens [1, T, ...], sequence n
    is tokens cu_seqlens[n] .. cu_seqlens[n + 1]).  cu_seqlens: int32, N + 1
    offsets, on the CPU or the GPU (the other copy is made here).  Returns
    (o [1,T,HV,DV] fp32, final_state [N,HV,DK,DV] fp32).  Heads, state layout
    and transforms as fwd_chunked; ``workspace`` (None: allocated here) holds
    every chunk's record, kda_fwd_chunked_varlen_workspace_bytes of them."""
    B, T, H, HV, DK, DV, dev, kind = _prep_fwd(q, k, v, beta, decay, None)
    tf = _transforms(kind, HV, DK, dev, use_gate_in_kernel, A_log, dt_bias, lower_bound,
                     use_beta_sigmoid_in_kernel, allow_neg_eigval)
    if B != 1:
        raise ValueError("packed sequences need B == 1")
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens must be a 1-D tensor of N + 1 offsets")
    N = cu_seqlens.numel() - 1
    cu_host = cu_seqlens.to("cpu", torch.int32).contiguous()
    cu_dev = cu_seqlens.to(dev, torch.int32).contiguous()
    sshape = _state_shape(N, HV, DK, DV, state_v_first)
    _check_state("initial_state", initial_state, sshape, dev)
    o = out if out is not None else torch.empty((1, T, HV, DV), device=dev, dtype=torch.float32)
    _check_state("out", o, (1, T, HV, DV), dev)
    fs = final_state if final_state is not None else torch.empty(sshape, device=dev,
                                                                 dtype=torch.float32)
    _check_state("final_state", fs, sshape, dev)
    need = lib().kda_fwd_chunked_varlen_workspace_bytes(_ptr(cu_host), N, H, HV, DK, DV,
                                                        _dtype_code(q), kind, int(chunk_size))
    ws = _workspace(workspace, need, dev)
    st = lib().kda_fwd_chunked_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(decay), kind,
                                      _ptr(initial_state), _ptr(o), _ptr(fs), _ptr(cu_dev),
                                      _ptr(cu_host), N, T, H, HV, DK, DV, _dtype_code(q),
                                      _scale(softmax_scale), int(bool(use_qk_l2norm)),
                                      int(bool(state_v_first)), int(chunk_size), *tf,
                                      _ptr(ws), ws.numel() * ws.element_size(), _stream(dev))
    if st != 0:
        raise KdaError("kda_fwd_chunked_varlen", st)
    return o, fs


def fwd_recurrent(q, k, v, beta, decay=None, initial_state=None, softmax_scale=None,
                  use_qk_l2norm=True, out=None, final_state=None, state_v_first=False,
                  use_gate_in_kernel=False, A_log=None, dt_bias=None,
                lower_bound=None, use_beta_sigmoid_in_kernel=False, allow_neg_eigval=False):
    """Recurrent (sequential) forward.  Same arguments and returns as fwd_chunked."""
    B, T, H, HV, DK, DV, dev, kind = _prep_fwd(q, k, v, beta, decay, initial_state, state_v_first)
    tf = _transforms(kind, HV, DK, dev, use_gate_in_kernel, A_log, dt_bias, lower_bound,
                     use_beta_sigmoid_in_kernel, allow_neg_eigval)
    sshape = _state_shape(B, HV, DK, DV, state_v_first)
    o = out if out is not None else torch.empty((B, T, HV, DV), device=dev, dtype=torch.float32)
    _check_state("out", o, (B, T, HV, DV), dev)
    fs = final_state if final_state is not None else torch.empty(sshape, device=dev,
                                                                 dtype=torch.float32)
    _check_state("final_state", fs, sshape, dev)
    st = lib().kda_fwd_recurrent(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(decay), kind,
                                 _ptr(initial_state), _ptr(o), _ptr(fs), B, T, H, HV, DK, DV,
                                 _dtype_code(q), _scale(softmax_scale), int(bool(use_qk_l2norm)),
                                 int(bool(state_v_first)), *tf, _stream(dev))
    if st != 0:
        raise KdaError("kda_fwd_recurrent", st)
    return o, fs


def decode_step(q, k, v, beta, decay, state, softmax_scale=None, use_qk_l2norm=True, out=None,
                state_v_first=False, use_gate_in_kernel=False, A_log=None, dt_bias=None,
                lower_bound=None, use_beta_sigmoid_in_kernel=False, allow_neg_eigval=False):
    """One decode step for every (batch, value head): q, k [B,H,DK]; v [B,HV,DV];
    beta [B,HV]; decay None, [B,HV] or [B,HV,DK]; ``state`` [B,HV,DK,DV] fp32
    ([B,HV,DV,DK] with ``state_v_first``) is updated in place.  Returns
    o [B,HV,DV] fp32.  Transforms as fwd_chunked."""
    if q.dim() != 3 or v.dim() != 3:
        raise ValueError("q must be [B, H, DK] and v [B, HV, DV]")
    B, H, DK = q.shape
    HV, DV = v.shape[1], v.shape[2]
    dev, dt = q.device, q.dtype
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU device")
    _check_act("q", q, (B, H, DK), dt, dev)
    _check_act("k", k, (B, H, DK), dt, dev)
    _check_act("v", v, (B, HV, DV), dt, dev)
    _check_act("beta", beta, (B, HV), dt, dev)
    kind = _decay_kind(decay, (B, HV), DK)
    if decay is not None:
        _check_act("decay", decay, tuple(decay.shape), dt, dev)
    if state is None:
        raise ValueError("state is required")
    sshape = _state_shape(B, HV, DK, DV, state_v_first)
    _check_state("state", state, sshape, dev)
    o = out if out is not None else torch.empty((B, HV, DV), device=dev, dtype=torch.float32)
    _check_state("out", o, (B, HV, DV), dev)
    tf = _transforms(kind, HV, DK, dev, use_gate_in_kernel, A_log, dt_bias, lower_bound,
                     use_beta_sigmoid_in_kernel, allow_neg_eigval)
    st = lib().kda_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(decay), kind,
                               _ptr(state), _ptr(o), B, H, HV, DK, DV, _dtype_code(q),
                               _scale(softmax_scale), int(bool(use_qk_l2norm)),
                               int(bool(state_v_first)), *tf, _stream(dev))
    if st != 0:
        raise KdaError("kda_decode_step", st)
    return o


def bwd(q, k, v, beta, decay, initial_state, d_o, d_final_state=None, softmax_scale=None,
        use_qk_l2norm=True, workspace=None, with_initial_state_grad=True, state_v_first=False,
        use_gate_in_kernel=False, A_log=None, dt_bias=None, lower_bound=None,
        use_beta_sigmoid_in_kernel=False, allow_neg_eigval=False):
    """Gradients of fwd_chunked / fwd_recurrent's (o, final_state) with the same
    inputs and arguments, pulled back from d_o [B,T,HV,DV] and d_final_state
    (the state's shape; None: zeros), both fp32.  Returns a dict: dq, dk
    [B,T,H,DK], dv [B,T,HV,DV], dbeta [B,T,HV] (of the logits with
    ``use_beta_sigmoid_in_kernel``), ddecay (None or the decay's shape; of the
    raw gate with ``use_gate_in_kernel``), d_initial_state (None unless
    asked), dA_log [HV] and ddt_bias (dt_bias's shape) with
    ``use_gate_in_kernel`` (else None), all fp32.
    ``workspace``: kda_bwd_workspace_bytes of device memory (None: allocated)."""
    B, T, H, HV, DK, DV, dev, kind = _prep_fwd(q, k, v, beta, decay, initial_state, state_v_first)
    tf = _transforms(kind, HV, DK, dev, use_gate_in_kernel, A_log, dt_bias, lower_bound,
                     use_beta_sigmoid_in_kernel, allow_neg_eigval)
    sshape = _state_shape(B, HV, DK, DV, state_v_first)
    _check_state("d_o", d_o, (B, T, HV, DV), dev)
    if d_o is None:
        raise ValueError("d_o is required")
    _check_state("d_final_state", d_final_state, sshape, dev)
    f32 = dict(device=dev, dtype=torch.float32)
    dq = torch.empty((B, T, H, DK), **f32)
    dk = torch.empty((B, T, H, DK), **f32)
    dv = torch.empty((B, T, HV, DV), **f32)
    dbeta = torch.empty((B, T, HV), **f32)
    ddecay = None if decay is None else torch.empty(tuple(decay.shape), **f32)
    dinit = torch.empty(sshape, **f32) if with_initial_state_grad else None
    dA = torch.empty((HV,), **f32) if use_gate_in_kernel else None
    dbias = (torch.empty(tuple(dt_bias.shape), **f32)
             if use_gate_in_kernel and dt_bias is not None else None)
    need = lib().kda_bwd_workspace_bytes(B, T, HV, DK, DV)
    ws = _workspace(workspace, need, dev)
    st = lib().kda_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(decay), kind,
                       _ptr(initial_state), _ptr(d_o), _ptr(d_final_state), _ptr(dq), _ptr(dk),
                       _ptr(dv), _ptr(dbeta), _ptr(ddecay), _ptr(dinit), B, T, H, HV, DK, DV,
                       _dtype_code(q), _scale(softmax_scale), int(bool(use_qk_l2norm)),
                       int(bool(state_v_first)), *tf, _ptr(dA), _ptr(dbias),
                       _ptr(ws), ws.numel() * ws.element_size(), _stream(dev))
    if st != 0:
        raise KdaError("kda_bwd", st)
    return dict(dq=dq, dk=dk, dv=dv, dbeta=dbeta, ddecay=ddecay, d_initial_state=dinit,
                dA_log=dA, ddt_bias=dbias)
