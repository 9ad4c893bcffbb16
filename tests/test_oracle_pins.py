"""CPU tests: the oracle against what the pages and mathematics fix."""

import json
import os

import numpy as np
import pytest

import oracle.scan as scan_mod
from oracle import kda_chunked_ref, kda_decode, kda_scan, kda_scan_heads

import pins

TOL = 1e-12
_TRUE_STEP = scan_mod.recurrence_step


@pytest.mark.parametrize("pin", pins.PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    assert pin(kda_scan) < TOL


def test_chunked_ref_matches_scan():
    assert pins.pin_chunked_equals_scan(kda_scan, kda_chunked_ref) < 1e-10


def test_decode_is_single_step():
    rng = np.random.default_rng(3)
    B, H, D = 3, 2, 8
    q, k, v = (rng.standard_normal((B, H, D)) for _ in range(3))
    beta = rng.random((B, H))
    g = -rng.random((B, H))
    S = rng.standard_normal((B, H, D, D))
    o, S1 = kda_decode(q, k, v, beta, g, S)
    o2, S2 = kda_scan(q[:, None], k[:, None], v[:, None], beta[:, None], g[:, None], S)
    assert np.abs(o - o2[:, 0]).max() == 0 and np.abs(S1 - S2).max() == 0


def test_head_sample_matches_full():
    rng = np.random.default_rng(4)
    q, k, v, beta, g, S0 = pins._inputs(rng, 2, 10, 3, 4, 5, "channel")
    o, S = kda_scan(q, k, v, beta, g, S0)
    heads = [(1, 2), (0, 1)]
    os_, Ss = kda_scan_heads(q, k, v, beta, g, S0, heads)
    for i, (b, h) in enumerate(heads):
        assert np.abs(os_[i] - o[b, :, h]).max() < 1e-14
        assert np.abs(Ss[i] - S[b, h]).max() < 1e-14


def test_example_output_shape():
    """The ejkernel page's worked example prints only the output shape."""
    path = os.path.join(os.path.dirname(__file__), "golden", "ejkernel_example_shape.json")
    with open(path) as f:
        fx = json.load(f)
    B, T, H, D = fx["batch"], fx["seq_len"], fx["num_heads"], fx["head_dim"]
    rng = np.random.default_rng(0)
    q, k, v = (rng.standard_normal((B, T, H, D)) for _ in range(3))
    beta = 1 / (1 + np.exp(-rng.standard_normal((B, T, H))))
    decay = rng.standard_normal((B, T, H)) * -0.01
    o, S = kda_chunked_ref(q, k, v, beta, decay, chunk_size=fx["chunk_size"])
    assert list(o.shape) == fx["output_shape"]
    assert list(S.shape) == [B, H, D, D]
    o2, S2 = kda_scan(q, k, v, beta, decay)
    assert np.abs(o - o2).max() < 1e-10


# ---- planted mistakes: each broken copy of the step must fail some pin ----

def _step_decay_then_read(S, q_hat, k_hat, v, beta, gate):
    Sd = S if gate is None else gate[..., :, None] * S
    read = np.einsum("bhcn,bhc->bhn", Sd, k_hat)
    delta = beta[..., None] * (v - read)
    S_new = Sd + k_hat[..., :, None] * delta[..., None, :]
    return np.einsum("bhcn,bhc->bhn", S_new, q_hat), S_new


def _step_gate_on_value_axis(S, q_hat, k_hat, v, beta, gate):
    read = np.einsum("bhcn,bhc->bhn", S, k_hat)
    delta = beta[..., None] * (v - read)
    if gate is not None:
        dv = S.shape[-1]
        g = gate[..., :dv] if gate.shape[-1] >= dv else np.resize(gate, S.shape[:2] + (dv,))
        S = S * g[..., None, :]
    S_new = S + k_hat[..., :, None] * delta[..., None, :]
    return np.einsum("bhcn,bhc->bhn", S_new, q_hat), S_new


def _step_output_reads_old_state(S, q_hat, k_hat, v, beta, gate):
    o_old = np.einsum("bhcn,bhc->bhn", S, q_hat)
    _, S_new = _TRUE_STEP(S, q_hat, k_hat, v, beta, gate)
    return o_old, S_new


def _step_sign_flip(S, q_hat, k_hat, v, beta, gate):
    read = np.einsum("bhcn,bhc->bhn", S, k_hat)
    delta = beta[..., None] * (v + read)
    Sd = S if gate is None else gate[..., :, None] * S
    S_new = Sd + k_hat[..., :, None] * delta[..., None, :]
    return np.einsum("bhcn,bhc->bhn", S_new, q_hat), S_new


def _step_beta_outside(S, q_hat, k_hat, v, beta, gate):
    read = np.einsum("bhcn,bhc->bhn", S, k_hat)
    delta = beta[..., None] * v - read
    Sd = S if gate is None else gate[..., :, None] * S
    S_new = Sd + k_hat[..., :, None] * delta[..., None, :]
    return np.einsum("bhcn,bhc->bhn", S_new, q_hat), S_new


def _step_no_decay(S, q_hat, k_hat, v, beta, gate):
    return _TRUE_STEP(S, q_hat, k_hat, v, beta, None)


MUTANTS = [_step_decay_then_read, _step_gate_on_value_axis, _step_output_reads_old_state,
           _step_sign_flip, _step_beta_outside, _step_no_decay]


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda m: m.__name__)
def test_pins_catch_planted_mistakes(monkeypatch, mutant):
    monkeypatch.setattr(scan_mod, "recurrence_step", mutant)
    failures = []
    for pin in pins.PINS:
        try:
            err = pin(kda_scan)
        except Exception:  # a shape error also counts as caught
            err = np.inf
        if not err < TOL:
            failures.append(pin.__name__)
    assert failures, f"no pin caught {mutant.__name__}"


def test_value_heads_share_their_groups_qk_head():
    # grouped value heads (HV = 2H): value heads 2j and 2j + 1 read q/k head j,
    # so with the same v, beta, decay and state they give the same output,
    # while heads of different groups (2j, 2j + 2) do not
    rng = np.random.default_rng(11)
    B, T, H, DK, DV = 1, 9, 2, 8, 4
    q, k = rng.normal(size=(B, T, H, DK)), rng.normal(size=(B, T, H, DK))
    v1 = rng.normal(size=(B, T, 1, DV))
    v = np.repeat(v1, 2 * H, axis=2)
    beta = np.full((B, T, 2 * H), 0.7)
    decay = np.repeat(-rng.uniform(0.01, 0.3, size=(B, T, 1)), 2 * H, axis=2)
    o, S = kda_scan(q, k, v, beta, decay)
    assert np.max(np.abs(o[:, :, 0] - o[:, :, 1])) == 0.0
    assert np.max(np.abs(o[:, :, 2] - o[:, :, 3])) == 0.0
    assert np.max(np.abs(o[:, :, 0] - o[:, :, 2])) > 1e-3
    # and HV = H is the plain scan, head by head
    o1, _ = kda_scan(q[:, :, 1:2], k[:, :, 1:2], v[:, :, 2:3], beta[:, :, 2:3], decay[:, :, 2:3])
    assert np.max(np.abs(o1[:, :, 0] - o[:, :, 2])) < 1e-14


def test_head_sample_with_grouped_value_heads():
    # the sampled-head scan reads the q/k head of each value head
    rng = np.random.default_rng(12)
    B, T, H, HV, DK, DV = 2, 7, 2, 6, 8, 4
    q, k = rng.normal(size=(B, T, H, DK)), rng.normal(size=(B, T, H, DK))
    v = rng.normal(size=(B, T, HV, DV))
    beta = rng.uniform(0.1, 0.9, size=(B, T, HV))
    decay = -rng.uniform(0.01, 0.3, size=(B, T, HV))
    o, S = kda_scan(q, k, v, beta, decay)
    heads = [(0, 0), (1, 4), (0, 2), (1, 5)]
    o_s, S_s = kda_scan_heads(q, k, v, beta, decay, None, heads)
    for i, (b, h) in enumerate(heads):
        assert np.max(np.abs(o_s[i] - o[b, :, h])) < 1e-14
        assert np.max(np.abs(S_s[i] - S[b, h])) < 1e-14


# ---- planted mistakes in the query scale and the L2 norm ----

def _scale_taken_literally(softmax_scale, dk):
    return dk ** -0.5 if softmax_scale is None else float(softmax_scale)


def _scale_nan_only_default(softmax_scale, dk):
    # non-positive values taken literally, only NaN and None mean the default
    if softmax_scale is None or softmax_scale != softmax_scale:
        return dk ** -0.5
    return float(softmax_scale)


def _l2_eps_added(x, eps=1e-12):
    return x / (np.sqrt(np.sum(x * x, axis=-1, keepdims=True)) + eps)


def _l2_no_floor(x, eps=1e-12):
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return np.divide(x, n, out=np.zeros_like(x), where=n > 0)


def _l2_floor_too_large(x, eps=1e-12):
    return x / np.maximum(np.sqrt(np.sum(x * x, axis=-1, keepdims=True)), 1e-6)


PREP_MUTANTS = [("resolve_scale", _scale_taken_literally), ("resolve_scale", _scale_nan_only_default),
                ("l2_normalize", _l2_eps_added), ("l2_normalize", _l2_no_floor),
                ("l2_normalize", _l2_floor_too_large)]


@pytest.mark.parametrize("attr,mutant", PREP_MUTANTS, ids=lambda m: getattr(m, "__name__", m))
def test_pins_catch_planted_prep_mistakes(monkeypatch, attr, mutant):
    monkeypatch.setattr(scan_mod, attr, mutant)
    failures = []
    for pin in pins.PINS:
        try:
            err = pin(kda_scan)
        except Exception:
            err = np.inf
        if not err < TOL:
            failures.append(pin.__name__)
    assert failures, f"no pin caught {mutant.__name__}"
