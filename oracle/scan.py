"""Plain fp64 CPU oracle for the gated delta-rule forward pass.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import this module;
only the tests, the smoke check and the CPU-baseline leg of the benchmark do.
It shares no code with the HIP library.

What it computes (ejkernel "kernel_delta_attention._interface", section
"Kernel Delta Attention", the core recurrence and its parameter list):

    h_t = exp(decay_t) * h_{t-1} + k_t (beta_t * (v_t - h_{t-1}^T k_t))^T
    o_t = h_t^T q_t

with h_t a [DK, DV] state per (batch, head), indexed (key channel, value
channel).  The readings taken where the page is terse:

* the delta term reads the previous state *before* it is decayed, exactly as
  the printed recurrence has it (h_{t-1}, not exp(decay_t) h_{t-1});
* ``h @ k`` and ``h @ q`` contract over the key channel (the state is
  [head_dim, value_dim]), i.e. h^T k and h^T q;
* the output reads the *updated* state h_t;
* with ``use_qk_l2norm`` q and k are divided by max(||x||_2, 1e-12) first, and
  q is then multiplied by ``softmax_scale`` (default DK**-0.5; a value that is
  None, NaN or <= 0 means the default);
* ``decay`` may be None (no decay), one log-space value per (token, head), or
  one per (token, head, key channel) -- the per-key-channel gate of the TileOPs
  "Kimi Delta Attention" operator, which scales the rows of the state indexed
  by key channel (TileOPs "Linear Attention Operators", GLARecurrentFwdOp,
  S_new = diag(exp(gk)) S + ...);
* beta is used as given (TileOPs DeltaNetFwdOp: beta is already transformed).

Everything is computed in float64 from the exact values the caller passes.
"""

from __future__ import annotations

import math

import numpy as np

L2_EPS = 1e-12


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):  # a torch tensor: read its exact values
        x = x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def resolve_scale(softmax_scale, dk):
    """Query scale: DK**-0.5 unless a positive finite value is given
    (ejkernel kda parameter list, softmax_scale; TileOPs GLA ops treat a
    non-positive scale as the default)."""
    if softmax_scale is None:
        return dk ** -0.5
    s = float(softmax_scale)
    if not math.isfinite(s) or s <= 0.0:
        return dk ** -0.5
    return s


def l2_normalize(x, eps=L2_EPS):
    """x / max(||x||_2, eps) along the last axis (kda-neuron-kernels README,
    'Input contract': the caller L2-normalises q and k along the head dim)."""
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / np.maximum(n, eps)


def prepare_qk(q, k, softmax_scale, use_qk_l2norm):
    """Return (q_hat * scale, k_hat): normalise first, then scale the query."""
    dk = q.shape[-1]
    if use_qk_l2norm:
        q = l2_normalize(q)
        k = l2_normalize(k)
    return q * resolve_scale(softmax_scale, dk), k


def _gate(decay_t, dk):
    """exp(decay) as a per-key-channel factor [..., DK] (or None)."""
    if decay_t is None:
        return None
    g = np.exp(decay_t)
    if g.ndim == 2:
        # one value per (batch, head): the same factor for every key channel
        g = np.broadcast_to(g[..., None], g.shape + (dk,))
    return g


def recurrence_step(S, q_hat, k_hat, v, beta, gate):
    """One step of the recurrence for every (batch, head) at once.

    S      [B, H, DK, DV]   previous state h_{t-1}
    q_hat  [B, H, DK]       normalised and scaled query
    k_hat  [B, H, DK]       normalised key
    v      [B, H, DV]
    beta   [B, H]
    gate   [B, H, DK] exp(decay_t) per key channel, or None
    Returns (o_t [B, H, DV], S_t).
    """
    read = np.einsum("bhcn,bhc->bhn", S, k_hat)          # h_{t-1}^T k_t
    delta = beta[..., None] * (v - read)                  # beta_t (v_t - h_{t-1}^T k_t)
    decayed = S if gate is None else gate[..., :, None] * S
    S_new = decayed + k_hat[..., :, None] * delta[..., None, :]
    o = np.einsum("bhcn,bhc->bhn", S_new, q_hat)          # h_t^T q_t
    return o, S_new


def expand_qk_heads(x, hv):
    """q or k [B, T, H, DK] -> [B, T, HV, DK] for HV recurrent heads, a
    multiple of H (TileOPs "Linear Attention Operators", GDNFwdOp and
    KDAFwdOp: q and k have H heads, v and the state HV).  The page does not
    say which q/k head a value head reads; the grouped reading is taken:
    value head hv reads q/k head hv // (HV // H), so consecutive value heads
    share one."""
    h = x.shape[2]
    if hv == h:
        return x
    if hv % h:
        raise ValueError(f"{hv} value heads is not a multiple of {h} q/k heads")
    return np.repeat(x, hv // h, axis=2)


def kda_scan(q, k, v, beta, decay=None, initial_state=None, softmax_scale=None,
             use_qk_l2norm=True):
    """Sequential fp64 scan of the recurrence over all tokens.

    q, k [B, T, H, DK]; v [B, T, HV, DV] (HV a multiple of H, see
    expand_qk_heads; HV = H is the plain case); beta [B, T, HV];
    decay None | [B, T, HV] | [B, T, HV, DK] (log space);
    initial_state None (zeros) | [B, HV, DK, DV].
    Returns (o [B, T, HV, DV], final_state [B, HV, DK, DV]) in float64.
    """
    q, k, v, beta = _f64(q), _f64(k), _f64(v), _f64(beta)
    q, k = expand_qk_heads(q, v.shape[2]), expand_qk_heads(k, v.shape[2])
    decay = _f64(decay)
    B, T, H, DK = q.shape
    DV = v.shape[-1]
    qh, kh = prepare_qk(q, k, softmax_scale, use_qk_l2norm)
    S = np.zeros((B, H, DK, DV)) if initial_state is None else _f64(initial_state).copy()
    o = np.zeros((B, T, H, DV))
    for t in range(T):
        gate = None if decay is None else _gate(decay[:, t], DK)
        o[:, t], S = recurrence_step(S, qh[:, t], kh[:, t], v[:, t], beta[:, t], gate)
    return o, S


def kda_decode(q, k, v, beta, decay, state, softmax_scale=None, use_qk_l2norm=True):
    """Single-step mode (ejkernel kda, 'Single-step: seq_len=1 with
    initial_state'): q, k [B, H, DK], v [B, H, DV], beta [B, H],
    decay None | [B, H] | [B, H, DK], state [B, H, DK, DV].
    Returns (o [B, H, DV], new_state) -- the scan with T = 1."""
    q, k, v, beta, decay = _f64(q), _f64(k), _f64(v), _f64(beta), _f64(decay)
    o, S = kda_scan(q[:, None], k[:, None], v[:, None], beta[:, None],
                    None if decay is None else decay[:, None],
                    initial_state=state, softmax_scale=softmax_scale,
                    use_qk_l2norm=use_qk_l2norm)
    return o[:, 0], S


def kda_scan_heads(q, k, v, beta, decay, initial_state, heads, softmax_scale=None,
                   use_qk_l2norm=True):
    """The scan restricted to a list of (b, h) pairs, h a value head: each
    head's recurrence is independent of every other head, so a sample of
    heads can be checked at full sequence length.  With HV value heads over H
    q/k heads, value head h reads q/k head h // (HV // H) (expand_qk_heads).
    Returns (o [n, T, DV], S [n, DK, DV])."""
    outs, states = [], []
    group = v.shape[2] // q.shape[2]
    for (b, h) in heads:
        sl = (slice(b, b + 1), slice(None), slice(h, h + 1))
        qsl = (slice(b, b + 1), slice(None), slice(h // group, h // group + 1))
        dec = None if decay is None else decay[sl]
        init = None if initial_state is None else initial_state[b:b + 1, h:h + 1]
        o, S = kda_scan(q[qsl], k[qsl], v[sl], beta[sl], dec, init, softmax_scale,
                        use_qk_l2norm)
        outs.append(o[0, :, 0])
        states.append(S[0, 0])
    return np.stack(outs), np.stack(states)
