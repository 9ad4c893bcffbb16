"""fp64 chunked (WY) form of the same recurrence -- TEST INFRASTRUCTURE ONLY.

This is not the oracle; ``oracle.scan.kda_scan`` is.  It restates the
"parallel within chunks, sequential across chunks" mode of ejkernel's kda
(section "Algorithm Modes") in the WY form that the TileOPs DeltaNet pipeline
names (prepare_wy_repr -> (Aw, Au) -> forward), written out for the gated
recurrence with the delta term reading the undecayed previous state.  The
tests pin it to the scan (the two must agree to rounding for every chunk
size), so the chunk algebra is checked on the CPU before any GPU code runs.

For one chunk of C tokens (rows r, s = 0..C-1), with S0 the state entering it,
G the inclusive in-chunk cumulative log decay per key channel and Gx the
exclusive one (Gx_r = G_{r-1}, Gx_0 = 0):

    A_rs = beta_r sum_c k_rc k_sc exp(Gx_rc - G_sc)        s < r, else 0
    Tm   = (I + A)^-1
    W    = Tm diag(beta) (K * exp(Gx))      U = Tm diag(beta) V
    D    = U - W S0                         (the per-token "v_new")
    O    = (Q * exp(G)) S0 + (mask_{s<=r} * P) D,
           P_rs = sum_c q_rc k_sc exp(G_rc - G_sc)
    S_C  = exp(G_last) * S0 + (K * exp(G_last - G))^T D

Derivation: unroll S_{r-1} = diag(exp(Gx_r)) S0 + sum_{s<r}
diag(exp(Gx_r - G_s)) k_s d_s^T inside the chunk, substitute it into
d_r = beta_r (v_r - S_{r-1}^T k_r) and o_r = S_r^T q_r, and collect the d's
on one side: (I + A) D = diag(beta) V - diag(beta) (K * exp(Gx)) S0.
"""

from __future__ import annotations

import numpy as np

from .scan import _f64, prepare_qk


def kda_chunked_ref(q, k, v, beta, decay=None, initial_state=None, softmax_scale=None,
                    use_qk_l2norm=True, chunk_size=64):
    q, k, v, beta = _f64(q), _f64(k), _f64(v), _f64(beta)
    decay = _f64(decay)
    B, T, H, DK = q.shape
    DV = v.shape[-1]
    qh, kh = prepare_qk(q, k, softmax_scale, use_qk_l2norm)
    if decay is None:
        g = np.zeros((B, T, H, DK))
    elif decay.ndim == 3:
        g = np.broadcast_to(decay[..., None], (B, T, H, DK))
    else:
        g = decay
    o = np.zeros((B, T, H, DV))
    S_all = np.zeros((B, H, DK, DV)) if initial_state is None else _f64(initial_state).copy()
    for b in range(B):
        for h in range(H):
            S = S_all[b, h].copy()
            for t0 in range(0, T, chunk_size):
                t1 = min(T, t0 + chunk_size)
                Q, K, V = qh[b, t0:t1, h], kh[b, t0:t1, h], v[b, t0:t1, h]
                bt = beta[b, t0:t1, h]
                G = np.cumsum(g[b, t0:t1, h], axis=0)            # inclusive
                Gx = np.vstack([np.zeros((1, DK)), G[:-1]])      # exclusive
                n = t1 - t0
                strict = np.tril(np.ones((n, n)), -1)
                incl = np.tril(np.ones((n, n)))
                # pairwise decayed Gram matrices; exponents are masked before exp
                ex_a = np.where(strict[..., None] > 0, Gx[:, None, :] - G[None, :, :], -np.inf)
                ex_p = np.where(incl[..., None] > 0, G[:, None, :] - G[None, :, :], -np.inf)
                A = bt[:, None] * np.einsum("rc,sc,rsc->rs", K, K, np.exp(ex_a))
                P = np.einsum("rc,sc,rsc->rs", Q, K, np.exp(ex_p))
                Tm = np.linalg.inv(np.eye(n) + A)
                W = Tm @ (bt[:, None] * K * np.exp(Gx))
                U = Tm @ (bt[:, None] * V)
                D = U - W @ S
                o[b, t0:t1, h] = (Q * np.exp(G)) @ S + P @ D
                S = np.exp(G[-1])[:, None] * S + (K * np.exp(G[-1][None, :] - G)).T @ D
            S_all[b, h] = S
    return o, S_all
