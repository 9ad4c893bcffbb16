"""Pins for the oracle: facts fixed by the pages or by mathematics, each written
independently of the oracle's own formula.

Every pin takes a ``scan`` callable with the signature of
``oracle.scan.kda_scan`` and returns the largest deviation it found, so the
same pins can be run against deliberately broken copies of the oracle (see
``test_oracle_pins.test_pins_catch_planted_mistakes``).
"""

from __future__ import annotations

import numpy as np


def _rng(seed):
    return np.random.default_rng(seed)


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _inputs(rng, B, T, H, DK, DV, decay="head"):
    q = rng.standard_normal((B, T, H, DK))
    k = rng.standard_normal((B, T, H, DK))
    v = rng.standard_normal((B, T, H, DV))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    if decay == "none":
        g = None
    elif decay == "head":
        g = -np.abs(rng.standard_normal((B, T, H))) * 0.4
    else:
        g = -np.abs(rng.standard_normal((B, T, H, DK))) * 0.4
    S0 = rng.standard_normal((B, H, DK, DV)) * 0.3
    return q, k, v, beta, g, S0


def pin_single_step_closed_form(scan):
    """One step in closed form.  The ungated step printed on the TileOPs page
    (DeltaNetRecurrentFwdOp: v_new = beta (v - S k), o = S q + (q.k) v_new,
    S_new = S + outer(k, v_new)), with the gate of the ejkernel recurrence
    applied to the state: the output is read from the old state plus a
    rank-one correction, not from the updated state."""
    worst = 0.0
    for decay in ("none", "head", "channel"):
        rng = _rng(11)
        q, k, v, beta, g, S0 = _inputs(rng, 2, 1, 3, 6, 5, decay)
        scale = 0.37
        o, S = scan(q, k, v, beta, g, S0, softmax_scale=scale, use_qk_l2norm=True)
        qh, kh = _unit(q[:, 0]) * scale, _unit(k[:, 0])
        if g is None:
            e = np.ones(qh.shape)
        elif g.ndim == 3:
            e = np.repeat(np.exp(g[:, 0])[..., None], 6, axis=-1)
        else:
            e = np.exp(g[:, 0])
        for b in range(2):
            for h in range(3):
                Sm = S0[b, h]
                v_new = beta[b, 0, h] * (v[b, 0, h] - Sm.T @ kh[b, h])
                o_cf = Sm.T @ (e[b, h] * qh[b, h]) + (qh[b, h] @ kh[b, h]) * v_new
                S_cf = e[b, h][:, None] * Sm + np.outer(kh[b, h], v_new)
                worst = max(worst, np.abs(o_cf - o[b, 0, h]).max(), np.abs(S_cf - S[b, h]).max())
    return worst


def pin_beta_zero_readout(scan):
    """beta = 0: nothing is written, so the state is the initial state decayed
    by the running product of gates, and every output is a decayed readout of
    the initial state (zero when the initial state is zero)."""
    worst = 0.0
    for decay in ("none", "head", "channel"):
        rng = _rng(12)
        q, k, v, beta, g, S0 = _inputs(rng, 1, 9, 2, 4, 3, decay)
        beta = np.zeros_like(beta)
        o, S = scan(q, k, v, beta, g, S0, softmax_scale=1.0, use_qk_l2norm=True)
        qh = _unit(q)
        if g is None:
            G = np.zeros(q.shape)
        elif g.ndim == 3:
            G = np.repeat(np.cumsum(g, axis=1)[..., None], 4, axis=-1)
        else:
            G = np.cumsum(g, axis=1)
        for h in range(2):
            for t in range(9):
                St = np.exp(G[0, t, h])[:, None] * S0[0, h]
                worst = max(worst, np.abs(St.T @ qh[0, t, h] - o[0, t, h]).max())
            worst = max(worst, np.abs(np.exp(G[0, -1, h])[:, None] * S0[0, h] - S[0, h]).max())
        o0, S_0 = scan(q, k, v, beta, g, np.zeros_like(S0), softmax_scale=1.0)
        worst = max(worst, np.abs(o0).max(), np.abs(S_0).max())
    return worst


def pin_orthonormal_keys_linear_attention(scan):
    """Ungated, beta = 1, zero initial state, orthonormal keys: every read
    S^T k_t is zero, so the rule reduces to causal linear attention,
    o_t = sum_{i<=t} (q_t . k_i) v_i (computed here by brute force)."""
    rng = _rng(13)
    T, DK, DV = 7, 8, 5
    Qm, _ = np.linalg.qr(rng.standard_normal((DK, DK)))
    k = Qm[:T][None, :, None, :]            # [1, T, 1, DK], rows orthonormal
    q = rng.standard_normal((1, T, 1, DK))
    v = rng.standard_normal((1, T, 1, DV))
    beta = np.ones((1, T, 1))
    o, S = scan(q, k, v, beta, None, None, softmax_scale=1.0, use_qk_l2norm=True)
    qh = _unit(q[0, :, 0])
    worst = 0.0
    for t in range(T):
        ref = sum((qh[t] @ k[0, i, 0]) * v[0, i, 0] for i in range(t + 1))
        worst = max(worst, np.abs(ref - o[0, t, 0]).max())
    ref_S = sum(np.outer(k[0, i, 0], v[0, i, 0]) for i in range(T))
    return max(worst, np.abs(ref_S - S[0, 0]).max())


def pin_overwrite(scan):
    """'The delta term computes what is new in v_t': ungated with beta = 1, a
    write of value v under unit key k leaves S^T k = v whatever the state was,
    and a second write under the same key replaces the first."""
    rng = _rng(14)
    DK, DV = 6, 4
    kk = _unit(rng.standard_normal(DK))
    k = np.stack([kk, kk])[None, :, None, :]
    q = rng.standard_normal((1, 2, 1, DK))
    v = rng.standard_normal((1, 2, 1, DV))
    S0 = rng.standard_normal((1, 1, DK, DV))
    _, S1 = scan(q[:, :1], k[:, :1], v[:, :1], np.ones((1, 1, 1)), None, S0, use_qk_l2norm=True)
    _, S2 = scan(q, k, v, np.ones((1, 2, 1)), None, S0, use_qk_l2norm=True)
    return max(np.abs(S1[0, 0].T @ kk - v[0, 0, 0]).max(),
               np.abs(S2[0, 0].T @ kk - v[0, 1, 0]).max())


def pin_transfer_matrix(scan):
    """Brute-force expansion for T <= 4: the step is affine in the state,
    S_t = M_t S_{t-1} + beta_t k_t v_t^T with M_t = diag(exp(g_t)) - beta_t
    k_t k_t^T, so S_T = M_T..M_1 S_0 + sum_i M_T..M_{i+1} beta_i k_i v_i^T and
    o_t = S_t^T q_t.  Catches a wrong sign, a transposed operand, a gate on
    the wrong side of the read, or a dropped term."""
    worst = 0.0
    for decay in ("none", "head", "channel"):
        rng = _rng(15)
        T, DK, DV = 4, 5, 3
        q, k, v, beta, g, S0 = _inputs(rng, 1, T, 1, DK, DV, decay)
        o, S = scan(q, k, v, beta, g, S0, softmax_scale=0.8, use_qk_l2norm=True)
        qh, kh = _unit(q[0, :, 0]) * 0.8, _unit(k[0, :, 0])
        if g is None:
            D = [np.eye(DK) for _ in range(T)]
        elif g.ndim == 3:
            D = [np.exp(g[0, t, 0]) * np.eye(DK) for t in range(T)]
        else:
            D = [np.diag(np.exp(g[0, t, 0])) for t in range(T)]
        M = [D[t] - beta[0, t, 0] * np.outer(kh[t], kh[t]) for t in range(T)]
        for t in range(T):
            prod = np.eye(DK)
            for j in range(t, -1, -1):
                prod = prod @ M[j]
            St = prod @ S0[0, 0]
            for i in range(t + 1):
                tail = np.eye(DK)
                for j in range(t, i, -1):
                    tail = tail @ M[j]
                St = St + tail @ (beta[0, i, 0] * np.outer(kh[i], v[0, i, 0]))
            worst = max(worst, np.abs(St.T @ qh[t] - o[0, t, 0]).max())
        worst = max(worst, np.abs(St - S[0, 0]).max())
    return worst


def pin_chunked_equals_scan(scan, chunked):
    """The chunked mode computes the same function as the scan for any chunk
    size, including a ragged last chunk."""
    worst = 0.0
    for decay in ("none", "head", "channel"):
        rng = _rng(16)
        q, k, v, beta, g, S0 = _inputs(rng, 2, 37, 2, 8, 6, decay)
        o, S = scan(q, k, v, beta, g, S0)
        for C in (1, 4, 16, 32, 64):
            o2, S2 = chunked(q, k, v, beta, g, S0, chunk_size=C)
            worst = max(worst, np.abs(o - o2).max(), np.abs(S - S2).max())
    return worst


def pin_state_handoff(scan):
    """Prefill then continue: running the second half of a sequence from the
    final state of the first half gives the same outputs and final state as
    one run (ejkernel example 'Incremental inference')."""
    worst = 0.0
    for decay in ("none", "head", "channel"):
        rng = _rng(17)
        q, k, v, beta, g, S0 = _inputs(rng, 2, 20, 2, 6, 4, decay)
        o, S = scan(q, k, v, beta, g, S0)
        t1 = 13
        gs = (lambda a, b: None) if g is None else (lambda a, b: g[:, a:b])
        oa, Sa = scan(q[:, :t1], k[:, :t1], v[:, :t1], beta[:, :t1], gs(0, t1), S0)
        ob, Sb = scan(q[:, t1:], k[:, t1:], v[:, t1:], beta[:, t1:], gs(t1, 20), Sa)
        worst = max(worst, np.abs(np.concatenate([oa, ob], 1) - o).max(), np.abs(Sb - S).max())
    return worst


def pin_linearity(scan):
    """For fixed q, k, beta and gates the outputs and the final state are
    jointly linear in (v, S_0)."""
    rng = _rng(18)
    q, k, v, beta, g, S0 = _inputs(rng, 1, 11, 2, 5, 4, "channel")
    v2, S02 = rng.standard_normal(v.shape), rng.standard_normal(S0.shape)
    a, b = 0.7, -1.3
    o1, S1 = scan(q, k, v, beta, g, S0)
    o2, S2 = scan(q, k, v2, beta, g, S02)
    o3, S3 = scan(q, k, a * v + b * v2, beta, g, a * S0 + b * S02)
    return max(np.abs(a * o1 + b * o2 - o3).max(), np.abs(a * S1 + b * S2 - S3).max())


def pin_value_permutation(scan):
    """Value channels never mix: permuting them permutes the outputs and the
    columns of the state."""
    rng = _rng(19)
    q, k, v, beta, g, S0 = _inputs(rng, 1, 9, 2, 5, 6, "head")
    perm = rng.permutation(6)
    o, S = scan(q, k, v, beta, g, S0)
    op, Sp = scan(q, k, v[..., perm], beta, g, S0[..., perm])
    return max(np.abs(o[..., perm] - op).max(), np.abs(S[..., perm] - Sp).max())


def pin_scale(scan):
    """The scale multiplies the queries only: o is proportional to it and the
    state does not depend on q or the scale; the default is DK**-0.5."""
    rng = _rng(20)
    q, k, v, beta, g, S0 = _inputs(rng, 1, 8, 2, 9, 3, "head")
    o1, S1 = scan(q, k, v, beta, g, S0, softmax_scale=1.0)
    o2, S2 = scan(q, k, v, beta, g, S0, softmax_scale=0.25)
    od, Sd = scan(q, k, v, beta, g, S0, softmax_scale=None)
    oq, Sq = scan(rng.standard_normal(q.shape), k, v, beta, g, S0, softmax_scale=0.25)
    return max(np.abs(0.25 * o1 - o2).max(), np.abs(od - o1 / 3.0).max(),
               np.abs(S1 - S2).max(), np.abs(S1 - Sd).max(), np.abs(S1 - Sq).max())


def pin_l2norm_idempotent(scan):
    """Pre-normalised q and k give the same result with the in-kernel L2 norm
    switched on or off."""
    rng = _rng(21)
    q, k, v, beta, g, S0 = _inputs(rng, 1, 8, 2, 7, 3, "channel")
    q, k = _unit(q), _unit(k)
    o1, S1 = scan(q, k, v, beta, g, S0, use_qk_l2norm=True)
    o2, S2 = scan(q, k, v, beta, g, S0, use_qk_l2norm=False)
    return max(np.abs(o1 - o2).max(), np.abs(S1 - S2).max())


def pin_gate_plumbing(scan):
    """No decay equals an all-zero decay; a per-channel decay that is the same
    in every channel equals the per-head decay."""
    rng = _rng(22)
    q, k, v, beta, g, S0 = _inputs(rng, 1, 8, 2, 4, 3, "head")
    o0, S0_ = scan(q, k, v, beta, None, S0)
    oz, Sz = scan(q, k, v, beta, np.zeros_like(g), S0)
    oh, Sh = scan(q, k, v, beta, g, S0)
    oc, Sc = scan(q, k, v, beta, np.repeat(g[..., None], 4, axis=-1), S0)
    return max(np.abs(o0 - oz).max(), np.abs(S0_ - Sz).max(),
               np.abs(oh - oc).max(), np.abs(Sh - Sc).max())


def pin_one_hot_keys_gla(scan):
    """Distinct one-hot keys never read back what was written, so with a zero
    initial state the rule becomes gated linear attention as the TileOPs page
    prints its step (GLARecurrentFwdOp: S_new = diag(exp(gk)) S + outer(k, v),
    o = scale q^T S_new) with k scaled by beta.  Pins that a per-channel gate
    scales the state rows indexed by key channel."""
    rng = _rng(23)
    T, DK, DV = 6, 7, 4
    order = rng.permutation(DK)[:T]
    k = np.zeros((1, T, 1, DK))
    k[0, np.arange(T), 0, order] = 1.0
    q = rng.standard_normal((1, T, 1, DK))
    v = rng.standard_normal((1, T, 1, DV))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((1, T, 1))))
    gk = -np.abs(rng.standard_normal((1, T, 1, DK)))
    o, S = scan(q, k, v, beta, gk, None, softmax_scale=0.5, use_qk_l2norm=False)
    Sm = np.zeros((DK, DV))
    worst = 0.0
    for t in range(T):
        Sm = np.diag(np.exp(gk[0, t, 0])) @ Sm + np.outer(beta[0, t, 0] * k[0, t, 0], v[0, t, 0])
        worst = max(worst, np.abs(0.5 * q[0, t, 0] @ Sm - o[0, t, 0]).max())
    return max(worst, np.abs(Sm - S[0, 0]).max())


def pin_nonpositive_scale_means_default(scan):
    """A scale that is zero, negative or NaN means the default DK**-0.5
    (TileOPs "Linear Attention Operators", GLA ops: a non-positive scale
    selects the default; ejkernel kda parameter list: no scale given means
    the inverse square root of the head size).  Compared with the scan at an
    explicit DK**-0.5, and with queries pre-multiplied by it at scale 1."""
    rng = _rng(24)
    DK = 16
    q, k, v, beta, g, S0 = _inputs(rng, 1, 7, 2, DK, 3, "head")
    o_ref, S_ref = scan(q, k, v, beta, g, S0, softmax_scale=0.25)
    # the same through a pre-scaled query: the norm removes the factor, so
    # the query is normalised first and given to the scan without the norm
    qn, kn = _unit(q), _unit(k)
    o_pre, _ = scan(qn * 0.25, kn, v, beta, g, S0, softmax_scale=1.0, use_qk_l2norm=False)
    worst = np.abs(o_pre - o_ref).max()
    for s in (0.0, -1.0, -0.0, float("nan"), None):
        o, S = scan(q, k, v, beta, g, S0, softmax_scale=s)
        worst = max(worst, np.abs(o - o_ref).max(), np.abs(S - S_ref).max())
    return worst


def _torch_normalize(x):
    """torch.nn.functional.normalize(x, p=2, dim=-1), the routine the
    kda-neuron-kernels README names for the caller's L2 norm (its default
    eps is 1e-12), run on the CPU in float64."""
    import torch
    return torch.nn.functional.normalize(torch.from_numpy(x), p=2.0, dim=-1).numpy()


def pin_l2_floor_matches_library_normalize(scan):
    """The in-kernel L2 norm is the library routine F.normalize: rows of
    ordinary norm, of tiny norm (1e-9, still normalised to unit length), of
    norm below the 1e-12 floor (divided by the floor, not normalised) and
    all-zero rows (left zero) give the same result as q, k normalised by
    that routine and passed with the norm off.  A zero key writes nothing
    and a zero query reads nothing."""
    rng = _rng(25)
    q, k, v, beta, g, S0 = _inputs(rng, 1, 8, 2, 6, 3, "channel")
    q[0, 1, 0] *= 1e-9 / np.linalg.norm(q[0, 1, 0])
    k[0, 2, 1] *= 1e-9 / np.linalg.norm(k[0, 2, 1])
    q[0, 3, 1] *= 3e-13 / np.linalg.norm(q[0, 3, 1])
    k[0, 4, 0] *= 5e-13 / np.linalg.norm(k[0, 4, 0])
    q[0, 5, 0] = 0.0
    k[0, 6, 1] = 0.0
    o1, S1 = scan(q, k, v, beta, g, S0, softmax_scale=0.5, use_qk_l2norm=True)
    o2, S2 = scan(_torch_normalize(q), _torch_normalize(k), v, beta, g, S0, softmax_scale=0.5,
                  use_qk_l2norm=False)
    worst = max(np.abs(o1 - o2).max(), np.abs(S1 - S2).max())
    # the zero query reads nothing at its token
    worst = max(worst, np.abs(o1[0, 5, 0]).max())
    return worst


PINS = [
    pin_single_step_closed_form,
    pin_beta_zero_readout,
    pin_orthonormal_keys_linear_attention,
    pin_overwrite,
    pin_transfer_matrix,
    pin_state_handoff,
    pin_linearity,
    pin_value_permutation,
    pin_scale,
    pin_l2norm_idempotent,
    pin_gate_plumbing,
    pin_one_hot_keys_gla,
    pin_nonpositive_scale_means_default,
    pin_l2_floor_matches_library_normalize,
]
