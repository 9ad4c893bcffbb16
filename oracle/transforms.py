"""fp64 input transforms -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the CPU-baseline leg of the benchmark
use this module; the library and its binding never import it.

* ``kda_decay`` -- ejkernel ``kernel_delta_attention._interface.kda_decay``
  (its docstring's computation): the per-token log-space decay from a raw
  gate, A = -exp(A_log), decay = A * softplus(gate + dt_bias), Mamba-style.
  The TileOPs "Linear Attention Operators" page (GDNFwdOp and KDAFwdOp,
  ``use_gate_in_kernel``) names the same formula and adds ``lower_bound``,
  a floor of the forget gate in log space; the reading taken here is the
  plain one, decay = max(decay, lower_bound).
* ``beta_transform`` -- the same page's ``use_beta_sigmoid_in_kernel``
  (beta = sigmoid(beta)) and ``allow_neg_eigval`` (2 * sigmoid(beta)).

Shapes: the page prints A_log and dt_bias as [num_heads] for a per-head gate
[B, T, H].  For the per-key-channel gate [B, T, H, DK] A_log stays per head
and dt_bias is per head and channel, [H, DK] (the plainest extension: the
bias is added to the gate element by element).
"""

from __future__ import annotations

import numpy as np

from .scan import _f64


def softplus(x):
    """log(1 + exp(x)), written so that large |x| neither overflows nor
    cancels: max(x, 0) + log1p(exp(-|x|))."""
    x = np.asarray(x, dtype=np.float64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def kda_decay(gate, A_log, dt_bias=None, lower_bound=None, per_channel=False):
    """decay = -exp(A_log) * softplus(gate + dt_bias), floored at lower_bound.

    gate [..., H] (per-head gate) or, with per_channel, [..., H, DK];
    A_log [H]; dt_bias None (zeros) | [H] | [H, DK] matching the gate."""
    g = _f64(gate)
    A = -np.exp(_f64(A_log))
    if per_channel:
        A = A[:, None]          # one A per head, shared by its key channels
    if dt_bias is not None:
        g = g + _f64(dt_bias)
    d = A * softplus(g)
    if lower_bound is not None:
        d = np.maximum(d, float(lower_bound))
    return d


def beta_transform(beta, allow_neg_eigval=False):
    """sigmoid(beta), or 2 * sigmoid(beta) with allow_neg_eigval."""
    b = _f64(beta)
    with np.errstate(over="ignore"):
        s = 1.0 / (1.0 + np.exp(-b))
    return 2.0 * s if allow_neg_eigval else s
