"""CPU tests: the oracle's input transforms against closed forms.

kda_decay follows ejkernel's kda_decay (-exp(A_log) * softplus(gate +
dt_bias)); the floor and the beta transforms follow the TileOPs GDNFwdOp /
KDAFwdOp parameter lists.  Every pin below checks a value fixed by the
mathematics (softplus(log(e^m - 1)) = m, sigmoid(log 3) = 3/4, ...) rather
than a restatement of the formula, and the planted-mistake test shows that
each plausible slip in the transforms fails at least one pin.
"""

import math

import numpy as np
import pytest

from oracle import transforms as T

TOL = 1e-13


def _inv_softplus(m):
    """x with softplus(x) = m (m > 0): log(e^m - 1)."""
    return np.log(np.expm1(m))


def pin_example_zero_inputs(decay_fn, beta_fn):
    # the page's worked call: zero gate, A_log and dt_bias, shape [2, 10, 4];
    # softplus(0) = log 2 and A = -1, so every decay is -log 2 (and <= 0)
    d = decay_fn(np.zeros((2, 10, 4)), np.zeros(4), np.zeros(4))
    if d.shape != (2, 10, 4):
        return np.inf
    return float(np.max(np.abs(d + math.log(2.0))))


def pin_head_scale_and_bias(decay_fn, beta_fn):
    # A_log[h] = log(h + 1), gate + dt_bias = log(e^m - 1): decay = -(h + 1) m
    H = 3
    m = np.array([[0.25, 1.0, 3.0], [2.0, 0.5, 7.0]])          # [T, H]
    bias = np.array([0.5, -1.0, 2.0])
    gate = _inv_softplus(m) - bias
    d = decay_fn(gate[None], np.log(np.arange(1, H + 1)), bias)
    want = -(np.arange(1, H + 1)[None, None, :]) * m[None]
    return float(np.max(np.abs(d - want)))


def pin_channel_indexing(decay_fn, beta_fn):
    # per-channel gate: A per head, bias per (head, channel);
    # decay[t, h, c] = -(h + 1) (c + 1) from gate + bias = log(e^(c+1) - 1)
    H, DK = 2, 5
    m = np.broadcast_to(np.arange(1, DK + 1, dtype=np.float64), (H, DK))
    bias = np.arange(H * DK, dtype=np.float64).reshape(H, DK) * 0.1 - 0.3
    gate = np.broadcast_to(_inv_softplus(m) - bias, (1, 2, H, DK))
    d = decay_fn(gate, np.log(np.arange(1, H + 1, dtype=np.float64)), bias, per_channel=True)
    want = -np.arange(1, H + 1)[:, None] * np.arange(1, DK + 1)[None, :]
    return float(np.max(np.abs(d - want[None, None])))


def pin_softplus_limits(decay_fn, beta_fn):
    # softplus(x) -> x for large x and -> e^x for very negative x; A = -1
    x = np.array([[40.0, 700.0, -40.0, -700.0]])
    d = decay_fn(x, np.zeros(4), None)
    want = -np.array([[40.0, 700.0, math.exp(-40.0), math.exp(-700.0)]])
    return float(np.max(np.abs(d - want) / np.abs(want)))


def pin_softplus_identity(decay_fn, beta_fn):
    # softplus(x) - softplus(-x) = x, so decay(x) - decay(-x) = -x with A = -1
    x = np.linspace(-30, 30, 61)[None]
    return float(np.max(np.abs(decay_fn(x, np.zeros(61)) - decay_fn(-x, np.zeros(61)) + x)))


def pin_lower_bound(decay_fn, beta_fn):
    # A = -10, softplus = 1: decay -10; a floor at -4 lifts it, one at -20 does not
    gate = _inv_softplus(np.ones((1, 1)))
    a = decay_fn(gate, np.log([10.0]), None, lower_bound=-4.0)
    b = decay_fn(gate, np.log([10.0]), None, lower_bound=-20.0)
    return float(abs(a[0, 0] + 4.0) + abs(b[0, 0] + 10.0))


def pin_beta_sigmoid(decay_fn, beta_fn):
    b = np.array([0.0, math.log(3.0), -math.log(3.0), 800.0, -800.0])
    s = beta_fn(b)
    s2 = beta_fn(b, allow_neg_eigval=True)
    want = np.array([0.5, 0.75, 0.25, 1.0, 0.0])
    return float(np.max(np.abs(s - want)) + np.max(np.abs(s2 - 2 * want)))


PINS = [pin_example_zero_inputs, pin_head_scale_and_bias, pin_channel_indexing,
        pin_softplus_limits, pin_softplus_identity, pin_lower_bound, pin_beta_sigmoid]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_transform_pin(pin):
    assert pin(T.kda_decay, T.beta_transform) < TOL


def test_decay_is_non_positive():
    rng = np.random.default_rng(5)
    d = T.kda_decay(rng.normal(0, 5, (4, 64, 8)), rng.normal(0, 2, 8), rng.normal(0, 2, 8))
    assert np.all(d <= 0)


# ---- planted mistakes: each must fail at least one pin ----

def _sp(x):
    return np.log1p(np.exp(x))


def _m_no_exp(gate, A_log, dt_bias=None, lower_bound=None, per_channel=False):
    A = -np.asarray(A_log, float)
    A = A[:, None] if per_channel else A
    g = gate + (0 if dt_bias is None else dt_bias)
    d = A * _sp(g)
    return d if lower_bound is None else np.maximum(d, lower_bound)


def _m_bias_outside(gate, A_log, dt_bias=None, lower_bound=None, per_channel=False):
    A = -np.exp(A_log)
    A = A[:, None] if per_channel else A
    d = A * _sp(gate) + (0 if dt_bias is None else dt_bias)
    return d if lower_bound is None else np.maximum(d, lower_bound)


def _m_sign(gate, A_log, dt_bias=None, lower_bound=None, per_channel=False):
    return -T.kda_decay(gate, A_log, dt_bias, lower_bound, per_channel)


def _m_channel_A(gate, A_log, dt_bias=None, lower_bound=None, per_channel=False):
    # A indexed by the last axis (key channel) instead of the head
    A = -np.exp(np.resize(np.asarray(A_log, float), np.shape(gate)[-1]))
    g = gate + (0 if dt_bias is None else dt_bias)
    d = A * T.softplus(g)
    return d if lower_bound is None else np.maximum(d, lower_bound)


def _m_floor_as_cap(gate, A_log, dt_bias=None, lower_bound=None, per_channel=False):
    d = T.kda_decay(gate, A_log, dt_bias, None, per_channel)
    return d if lower_bound is None else np.minimum(d, lower_bound)


def _m_relu(gate, A_log, dt_bias=None, lower_bound=None, per_channel=False):
    # softplus replaced by max(x, 0)
    A = -np.exp(A_log)
    A = A[:, None] if per_channel else A
    d = A * np.maximum(gate + (0 if dt_bias is None else dt_bias), 0)
    return d if lower_bound is None else np.maximum(d, lower_bound)


def _b_tanh(b, allow_neg_eigval=False):
    s = np.tanh(np.asarray(b, float))
    return 2 * s if allow_neg_eigval else s


def _b_neg_ignored(b, allow_neg_eigval=False):
    return T.beta_transform(b)


DECAY_MUTANTS = [_m_no_exp, _m_bias_outside, _m_sign, _m_channel_A, _m_floor_as_cap, _m_relu]
BETA_MUTANTS = [_b_tanh, _b_neg_ignored]


def _caught(decay_fn, beta_fn):
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                err = pin(decay_fn, beta_fn)
        except Exception:  # a shape error counts as caught
            err = np.inf
        if not err < TOL:
            return True
    return False


@pytest.mark.parametrize("mutant", DECAY_MUTANTS, ids=lambda m: m.__name__)
def test_decay_pins_catch_planted_mistakes(mutant):
    assert _caught(mutant, T.beta_transform)


@pytest.mark.parametrize("mutant", BETA_MUTANTS, ids=lambda m: m.__name__)
def test_beta_pins_catch_planted_mistakes(mutant):
    assert _caught(T.kda_decay, mutant)
