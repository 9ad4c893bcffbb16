"""Plain fp64 CPU oracle of the gated delta-rule BACKWARD pass.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: nothing in the
product path may import it.  It shares no code with the HIP library.

What it computes: the gradients of the forward recurrence that
``oracle.scan.kda_scan`` evaluates (ejkernel "kernel_delta_attention.
_interface", the core recurrence) with respect to every input, given the
gradient of the output and of the final state.  The set of gradients is the
one the pages name for the backward operators: dq, dk, dv, dbeta (TileOPs
"Linear Attention Operators", DeltaNetChunkBwdOp), dg and the final-state
gradient as an input (GLAChunkBwdOp: do and the final-state gradient), and the
initial-state gradient (kda-neuron-kernels README, kda_chunk_step_exact_bwd:
dq, dk, dv, dg, dbeta, dstate_in).  The pages print no formula for it; it is
reverse-mode differentiation of the recurrence, written out by hand below in
the order the forward runs backwards (no autograd), one token at a time:

    forward   r = S^T k,  delta = beta (v - r),  S' = diag(a) S + k delta^T,
              o = S'^T q,  a = exp(g)
    reverse   dS' += q do^T;       dq  = S' do
              ddelta = dS'^T k;    dk  = dS' delta;    da = rowsum(dS' * S)
              dS  = diag(a) dS' - beta k ddelta^T;     dk += -beta S ddelta
              dbeta = ddelta . (v - r);   dv = beta ddelta;   dg = a * da

q and k here are the normalised (and, for q, scaled) vectors; the gradient
is then carried through x / max(||x||, 1e-12) and the scale to the raw
inputs.  A per-head decay gets the sum over key channels of a * da.  With HV
value heads over H q/k heads (value head hv reads q/k head hv // (HV/H)) the
q and k gradients of a group's value heads add up.
"""

from __future__ import annotations

import numpy as np

from .scan import L2_EPS, _f64, expand_qk_heads, resolve_scale


def _norm_bwd(x, dxh, scale, use_qk_l2norm, eps=L2_EPS):
    """Gradient of xh = scale * x / max(||x||, eps) (or scale * x without the
    norm) with respect to x, given the gradient dxh of xh."""
    if not use_qk_l2norm:
        return scale * dxh
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    big = n > eps
    nn = np.where(big, n, 1.0)
    xn = x / nn
    proj = np.sum(xn * dxh, axis=-1, keepdims=True)
    return np.where(big, scale * (dxh - xn * proj) / nn, scale * dxh / eps)


def _sum_groups(dx, h):
    """[B, T, HV, D] gradients of expanded q/k heads -> [B, T, H, D]."""
    hv = dx.shape[2]
    if hv == h:
        return dx
    return dx.reshape(dx.shape[0], dx.shape[1], h, hv // h, dx.shape[3]).sum(axis=3)


def reverse_step(dS, S_prev, S_new, r, qh, kh, v, beta, a, do):
    """One token of the reverse pass for every (batch, head).

    dS [B, H, DK, DV] gradient of the state after the token; S_prev, S_new
    the states before and after it; r = S_prev^T kh; qh, kh [B, H, DK] the
    normalised (scaled) query and key; v [B, H, DV]; beta [B, H]; a [B, H, DK]
    exp(decay) per key channel; do [B, H, DV].
    Returns (dS_prev, dqh, dkh, dv, dbeta, da)."""
    delta = beta[..., None] * (v - r)
    # o = S_new^T qh
    dS = dS + qh[..., :, None] * do[..., None, :]
    dqh = np.einsum("bhcn,bhn->bhc", S_new, do)
    # S_new = diag(a) S_prev + kh delta^T
    ddelta = np.einsum("bhcn,bhc->bhn", dS, kh)
    dkh = np.einsum("bhcn,bhn->bhc", dS, delta)
    da = np.sum(dS * S_prev, axis=-1)
    dS_prev = a[..., :, None] * dS
    # delta = beta (v - S_prev^T kh)
    dbeta = np.sum(ddelta * (v - r), axis=-1)
    dv = beta[..., None] * ddelta
    dr = -beta[..., None] * ddelta
    dS_prev = dS_prev + kh[..., :, None] * dr[..., None, :]
    dkh = dkh + np.einsum("bhcn,bhn->bhc", S_prev, dr)
    return dS_prev, dqh, dkh, dv, dbeta, da


def kda_scan_bwd(q, k, v, beta, decay, initial_state, do, d_final_state=None,
                 softmax_scale=None, use_qk_l2norm=True):
    """Gradients of kda_scan's (o, final_state) pulled back from (do, d_final_state).

    q, k [B, T, H, DK]; v [B, T, HV, DV]; beta [B, T, HV]; decay None |
    [B, T, HV] | [B, T, HV, DK]; initial_state None | [B, HV, DK, DV];
    do [B, T, HV, DV]; d_final_state None (zeros) | [B, HV, DK, DV].
    Returns a dict of float64 arrays: dq, dk [B, T, H, DK], dv [B, T, HV, DV],
    dbeta [B, T, HV], ddecay (None, or the decay's shape), d_initial_state
    [B, HV, DK, DV].
    """
    q, k, v, beta, do = _f64(q), _f64(k), _f64(v), _f64(beta), _f64(do)
    decay = _f64(decay)
    H = q.shape[2]
    HV = v.shape[2]
    qe, ke = expand_qk_heads(q, HV), expand_qk_heads(k, HV)
    B, T, _, DK = qe.shape
    DV = v.shape[-1]
    scale = resolve_scale(softmax_scale, DK)
    if use_qk_l2norm:
        qh = qe / np.maximum(np.sqrt(np.sum(qe * qe, -1, keepdims=True)), L2_EPS) * scale
        kh = ke / np.maximum(np.sqrt(np.sum(ke * ke, -1, keepdims=True)), L2_EPS)
    else:
        qh, kh = qe * scale, ke
    if decay is None:
        a = np.ones((B, T, HV, DK))
    elif decay.ndim == 3:
        a = np.repeat(np.exp(decay)[..., None], DK, axis=-1)
    else:
        a = np.exp(decay)

    # forward, keeping every state: states[t] enters token t, states[T] is final
    S = np.zeros((B, HV, DK, DV)) if initial_state is None else _f64(initial_state).copy()
    states = [S]
    reads = []
    for t in range(T):
        r = np.einsum("bhcn,bhc->bhn", S, kh[:, t])
        reads.append(r)
        delta = beta[:, t, :, None] * (v[:, t] - r)
        S = a[:, t, :, :, None] * S + kh[:, t, :, :, None] * delta[:, :, None, :]
        states.append(S)

    dqh = np.zeros_like(qh)
    dkh = np.zeros_like(kh)
    dv = np.zeros_like(v)
    dbeta = np.zeros_like(beta)
    da = np.zeros((B, T, HV, DK))
    dS = np.zeros((B, HV, DK, DV)) if d_final_state is None else _f64(d_final_state).copy()
    for t in range(T - 1, -1, -1):
        dS, dqh[:, t], dkh[:, t], dv[:, t], dbeta[:, t], da[:, t] = reverse_step(
            dS, states[t], states[t + 1], reads[t], qh[:, t], kh[:, t], v[:, t], beta[:, t],
            a[:, t], do[:, t])

    dq = _sum_groups(_norm_bwd(qe, dqh, scale, use_qk_l2norm), H)
    dk = _sum_groups(_norm_bwd(ke, dkh, 1.0, use_qk_l2norm), H)
    if decay is None:
        ddecay = None
    elif decay.ndim == 3:
        ddecay = np.sum(da * a, axis=-1)
    else:
        ddecay = da * a
    return dict(dq=dq, dk=dk, dv=dv, dbeta=dbeta, ddecay=ddecay, d_initial_state=dS)


def _sigmoid(x):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-x))


def transforms_bwd(gate, A_log, dt_bias, logits, ddecay, dbeta, lower_bound, per_channel,
                   allow_neg_eigval):
    """The chain rule through the transforms (see kda_scan_bwd_transforms)."""
    from .transforms import softplus
    s = _sigmoid(logits)
    dlogits = dbeta * s * (1.0 - s) * (2.0 if allow_neg_eigval else 1.0)
    x = gate + (0.0 if dt_bias is None else dt_bias)
    negA = -np.exp(A_log)
    if per_channel:
        negA = negA[:, None]
    raw = negA * softplus(x)
    live = np.ones_like(raw, dtype=bool) if lower_bound is None else raw >= float(lower_bound)
    dgate = np.where(live, ddecay * negA * _sigmoid(x), 0.0)
    contrib = np.where(live, ddecay * raw, 0.0)
    dA = contrib.sum(axis=(0, 1, 3)) if per_channel else contrib.sum(axis=(0, 1))
    return dict(dbeta_logits=dlogits, dgate=dgate, dA_log=dA,
                ddt_bias=None if dt_bias is None else dgate.sum(axis=(0, 1)))


def kda_scan_bwd_transforms(q, k, v, beta_logits, gate, A_log, initial_state, do,
                            d_final_state=None, dt_bias=None, lower_bound=None, per_channel=False,
                            allow_neg_eigval=False, softmax_scale=None, use_qk_l2norm=True):
    """Gradients with respect to the raw inputs of the in-kernel transforms
    (oracle.transforms: decay = max(-exp(A_log) softplus(gate + dt_bias),
    lower_bound), beta = sigmoid(logits) or twice it), by the chain rule
    through kda_scan_bwd's decay and beta gradients:

        dlogits = dbeta * s (1 - s) (times 2 with allow_neg_eigval), s = sigmoid(logits)
        where the floor is not taken:
          dgate = ddecay * (-exp(A_log)) * sigmoid(gate + dt_bias)
          dA_log = sum over tokens (and channels) of ddecay * decay
          ddt_bias = sum over batch and tokens of dgate
        where it is taken, the decay is the constant floor: no gradient.

    gate [B, T, HV] or (per_channel) [B, T, HV, DK]; A_log [HV]; dt_bias
    None | [HV] | [HV, DK].  Returns kda_scan_bwd's dict with dbeta and ddecay
    replaced by dbeta_logits, dgate, dA_log and ddt_bias (None without a
    bias)."""
    from .transforms import beta_transform, kda_decay
    g = _f64(gate)
    a_log = _f64(A_log)
    bias = None if dt_bias is None else _f64(dt_bias)
    decay = kda_decay(g, a_log, bias, lower_bound, per_channel=per_channel)
    logits = _f64(beta_logits)
    beta = beta_transform(logits, allow_neg_eigval)
    out = kda_scan_bwd(q, k, v, beta, decay, initial_state, do, d_final_state,
                       softmax_scale=softmax_scale, use_qk_l2norm=use_qk_l2norm)
    out.update(transforms_bwd(g, a_log, bias, logits, out.pop("ddecay"), out.pop("dbeta"),
                              lower_bound, per_channel, allow_neg_eigval))
    return out
