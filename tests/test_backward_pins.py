"""CPU pins of the fp64 backward oracle (oracle.backward.kda_scan_bwd) against
what mathematics fixes independently of its reverse pass:

* finite differences: central differences of the pinned forward oracle,
  L = <do, o> + <dS_T, S_T>, for every input (q, k, v, beta, both decay kinds,
  the initial state), grouped value heads, the L2 norm on and off;
* the adjoint identity: (o, S_T) is linear in (v, S_0) for fixed q, k, beta,
  decay, so L(v, S_0) = <dv, v> + <dS_0, S_0> exactly;
* the single-token closed form (T = 1), derived by hand in matrix form;
* no decay = an all-zero decay, with the decay gradient then a * da summed.

Planted mistakes in the reverse step and in the norm's backward must each
fail some pin.
"""

import numpy as np
import pytest

import oracle.backward as bwd_mod
from oracle import kda_scan, kda_scan_bwd  # noqa: F401

_TRUE_STEP = bwd_mod.reverse_step
_TRUE_NORM = bwd_mod._norm_bwd


def _inputs(rng, B, T, H, HV, DK, DV, decay):
    q = rng.standard_normal((B, T, H, DK))
    k = rng.standard_normal((B, T, H, DK))
    v = rng.standard_normal((B, T, HV, DV))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, HV))))
    if decay == "none":
        g = None
    elif decay == "head":
        g = -np.abs(rng.standard_normal((B, T, HV))) * 0.5
    else:
        g = -np.abs(rng.standard_normal((B, T, HV, DK))) * 0.5
    S0 = rng.standard_normal((B, HV, DK, DV)) * 0.3
    do = rng.standard_normal((B, T, HV, DV))
    dST = rng.standard_normal((B, HV, DK, DV))
    return dict(q=q, k=k, v=v, beta=beta, decay=g, initial_state=S0), do, dST


def _loss(x, do, dST, **kw):
    o, S = kda_scan(x["q"], x["k"], x["v"], x["beta"], x["decay"], x["initial_state"], **kw)
    return float(np.sum(o * do) + np.sum(S * dST))


def _grads(x, do, dST, **kw):
    return kda_scan_bwd(x["q"], x["k"], x["v"], x["beta"], x["decay"], x["initial_state"], do,
                        dST, **kw)


GRAD_OF = {"q": "dq", "k": "dk", "v": "dv", "beta": "dbeta", "decay": "ddecay",
           "initial_state": "d_initial_state"}


def pin_finite_differences():
    """Largest relative deviation of the oracle's gradients from central
    differences of the forward oracle, over sampled elements of every input."""
    worst = 0.0
    cases = [("none", 2, 2, True, None), ("head", 1, 2, True, 0.6), ("channel", 1, 1, True, None),
             ("channel", 2, 1, False, 0.9), ("head", 2, 2, False, None)]
    for n, (decay, H, G, l2, scale) in enumerate(cases):
        rng = np.random.default_rng(100 + n)
        x, do, dST = _inputs(rng, 1, 5, H, H * G, 4, 3, decay)
        if not l2:
            x["q"] = x["q"] / np.linalg.norm(x["q"], axis=-1, keepdims=True)
            x["k"] = x["k"] / np.linalg.norm(x["k"], axis=-1, keepdims=True)
        kw = dict(softmax_scale=scale, use_qk_l2norm=l2)
        gr = _grads(x, do, dST, **kw)
        h = 1e-6
        for name, gname in GRAD_OF.items():
            if x[name] is None:
                continue
            flat = x[name].reshape(-1)
            idx = rng.choice(flat.size, size=min(flat.size, 12), replace=False)
            for i in idx:
                keep = flat[i]
                flat[i] = keep + h
                lp = _loss(x, do, dST, **kw)
                flat[i] = keep - h
                lm = _loss(x, do, dST, **kw)
                flat[i] = keep
                fd = (lp - lm) / (2 * h)
                an = gr[gname].reshape(-1)[i]
                worst = max(worst, abs(fd - an) / max(1.0, abs(fd)))
    return worst


def pin_adjoint_identity():
    """(o, S_T) is linear in (v, S_0): <do, o> + <dS_T, S_T> = <dv, v> + <dS_0, S_0>."""
    worst = 0.0
    for n, decay in enumerate(("none", "head", "channel")):
        rng = np.random.default_rng(200 + n)
        x, do, dST = _inputs(rng, 2, 7, 2, 4, 5, 3, decay)
        gr = _grads(x, do, dST)
        lhs = _loss(x, do, dST)
        rhs = float(np.sum(gr["dv"] * x["v"]) + np.sum(gr["d_initial_state"] * x["initial_state"]))
        worst = max(worst, abs(lhs - rhs) / max(1.0, abs(lhs)))
    return worst


def pin_single_token_closed_form():
    """T = 1, no norm, scale 1, per-channel decay D = diag(exp(g)):
    o = S0^T D q + (q.k) delta, delta = beta (v - S0^T k), S1 = D S0 + k delta^T.
    With L = do.o + <W, S1> and e = (q.k) do + W^T k (the gradient of delta):
    dv = beta e, dbeta = (v - S0^T k).e, dS0 = D q do^T + D W - beta k e^T,
    dq = D S0 do + (delta.do) k, dk = (delta.do) q + W delta - beta S0 e,
    dg = exp(g) * (S0 do . q + rowsum(W * S0))."""
    rng = np.random.default_rng(300)
    x, do, dST = _inputs(rng, 1, 1, 1, 1, 5, 4, "channel")
    gr = _grads(x, do, dST, softmax_scale=1.0, use_qk_l2norm=False)
    q, k, v, beta = x["q"][0, 0, 0], x["k"][0, 0, 0], x["v"][0, 0, 0], x["beta"][0, 0, 0]
    g, S0, d, W = x["decay"][0, 0, 0], x["initial_state"][0, 0], do[0, 0, 0], dST[0, 0]
    D = np.diag(np.exp(g))
    delta = beta * (v - S0.T @ k)
    e = (q @ k) * d + W.T @ k
    ref = dict(dv=beta * e, dbeta=(v - S0.T @ k) @ e,
               d_initial_state=D @ np.outer(q, d) + D @ W - beta * np.outer(k, e),
               dq=D @ S0 @ d + (delta @ d) * k,
               dk=(delta @ d) * q + W @ delta - beta * S0 @ e,
               ddecay=np.exp(g) * ((S0 @ d) * q + np.sum(W * S0, axis=1)))
    worst = 0.0
    for name, r in ref.items():
        got = gr[name].reshape(r.shape)
        worst = max(worst, np.abs(got - r).max() / max(1.0, np.abs(r).max()))
    return worst


def pin_zero_decay_equals_no_decay():
    """decay None and an all-zero decay give the same gradients; the zero
    decay's gradient is then the sum over channels of S * dS per token."""
    rng = np.random.default_rng(400)
    x, do, dST = _inputs(rng, 1, 6, 2, 2, 4, 3, "none")
    g0 = _grads(x, do, dST)
    x["decay"] = np.zeros((1, 6, 2))
    gz = _grads(x, do, dST)
    worst = 0.0
    for name in ("dq", "dk", "dv", "dbeta", "d_initial_state"):
        worst = max(worst, np.abs(g0[name] - gz[name]).max())
    # against central differences of the per-head decay at zero
    h = 1e-6
    for t in (0, 3, 5):
        xp = dict(x, decay=x["decay"].copy())
        xp["decay"][0, t, 1] = h
        xm = dict(x, decay=x["decay"].copy())
        xm["decay"][0, t, 1] = -h
        fd = (_loss(xp, do, dST) - _loss(xm, do, dST)) / (2 * h)
        worst = max(worst, abs(fd - gz["ddecay"][0, t, 1]) / max(1.0, abs(fd)))
    return worst


PINS = [pin_finite_differences, pin_adjoint_identity, pin_single_token_closed_form,
        pin_zero_decay_equals_no_decay]
TOL = {"pin_finite_differences": 1e-7, "pin_adjoint_identity": 1e-12,
       "pin_single_token_closed_form": 1e-12, "pin_zero_decay_equals_no_decay": 1e-7}


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_backward_pin(pin):
    err = pin()
    print(f"{pin.__name__}: {err:.2e}")
    assert err < TOL[pin.__name__]


# ---- planted mistakes ----

def _m_dk_without_read_term(dS, S_prev, S_new, r, qh, kh, v, beta, a, do):
    out = list(_TRUE_STEP(dS, S_prev, S_new, r, qh, kh, v, beta, a, do))
    delta = beta[..., None] * (v - r)
    out[2] = np.einsum("bhcn,bhn->bhc", dS + qh[..., :, None] * do[..., None, :], delta)
    return tuple(out)


def _m_da_from_new_state(dS, S_prev, S_new, r, qh, kh, v, beta, a, do):
    return _TRUE_STEP(dS, S_new, S_new, r, qh, kh, v, beta, a, do)[:5] + \
        (np.sum((dS + qh[..., :, None] * do[..., None, :]) * S_new, axis=-1),)


def _m_state_grad_not_decayed(dS, S_prev, S_new, r, qh, kh, v, beta, a, do):
    return _TRUE_STEP(dS, S_prev, S_new, r, qh, kh, v, beta, np.ones_like(a), do)[:5] + \
        (_TRUE_STEP(dS, S_prev, S_new, r, qh, kh, v, beta, a, do)[5],)


def _m_dq_from_old_state(dS, S_prev, S_new, r, qh, kh, v, beta, a, do):
    out = list(_TRUE_STEP(dS, S_prev, S_new, r, qh, kh, v, beta, a, do))
    out[1] = np.einsum("bhcn,bhn->bhc", S_prev, do)
    return tuple(out)


def _m_dbeta_without_read(dS, S_prev, S_new, r, qh, kh, v, beta, a, do):
    out = list(_TRUE_STEP(dS, S_prev, S_new, r, qh, kh, v, beta, a, do))
    ddelta = np.einsum("bhcn,bhc->bhn", dS + qh[..., :, None] * do[..., None, :], kh)
    out[4] = np.sum(ddelta * v, axis=-1)
    return tuple(out)


def _m_norm_without_projection(x, dxh, scale, use_qk_l2norm, eps=1e-12):
    if not use_qk_l2norm:
        return scale * dxh
    n = np.maximum(np.sqrt(np.sum(x * x, axis=-1, keepdims=True)), eps)
    return scale * dxh / n


MUTANTS = [("reverse_step", _m_dk_without_read_term), ("reverse_step", _m_da_from_new_state),
           ("reverse_step", _m_state_grad_not_decayed), ("reverse_step", _m_dq_from_old_state),
           ("reverse_step", _m_dbeta_without_read), ("_norm_bwd", _m_norm_without_projection)]


@pytest.mark.parametrize("attr,mutant", MUTANTS, ids=lambda m: getattr(m, "__name__", m))
def test_backward_pins_catch_planted_mistakes(monkeypatch, attr, mutant):
    monkeypatch.setattr(bwd_mod, attr, mutant)
    caught = []
    for pin in PINS:
        try:
            err = pin()
        except Exception:
            err = np.inf
        if not err < TOL[pin.__name__]:
            caught.append(pin.__name__)
    assert caught, f"no pin caught {mutant.__name__}"


# ---- the transforms' backward ----

from oracle import beta_transform, kda_decay, kda_scan_bwd_transforms  # noqa: E402

_TRUE_TF = bwd_mod.transforms_bwd


def pin_transform_finite_differences():
    """Central differences of the forward oracle fed the oracle's own
    transforms (raw gate -> decay, logits -> beta), for the gate, the beta
    logits, A_log and dt_bias; per-head and per-channel gates, with and
    without the floor (a floor of -0.6 catches some of these decays), and the
    factor 2 of allow_neg_eigval."""
    worst = 0.0
    cases = [(False, None, False, True), (True, -0.6, True, True), (True, None, False, False),
             (False, -0.6, True, True)]
    for n, (per_channel, lb, neg, bias) in enumerate(cases):
        rng = np.random.default_rng(500 + n)
        B, T, H, DK, DV = 1, 5, 2, 4, 3
        q, k = rng.standard_normal((B, T, H, DK)), rng.standard_normal((B, T, H, DK))
        v = rng.standard_normal((B, T, H, DV))
        logits = rng.standard_normal((B, T, H))
        gate = rng.standard_normal((B, T, H, DK) if per_channel else (B, T, H))
        A_log = 0.3 * rng.standard_normal(H)
        dt_bias = (rng.uniform(-2, 0, (H, DK) if per_channel else H)) if bias else None
        S0 = 0.3 * rng.standard_normal((B, H, DK, DV))
        do, dST = rng.standard_normal((B, T, H, DV)), rng.standard_normal((B, H, DK, DV))
        x = dict(gate=gate, logits=logits, A_log=A_log, dt_bias=dt_bias)

        def loss(x):
            dec = kda_decay(x["gate"], x["A_log"], x["dt_bias"], lb, per_channel=per_channel)
            o, S = kda_scan(q, k, v, beta_transform(x["logits"], neg), dec, S0)
            return float(np.sum(o * do) + np.sum(S * dST))

        gr = kda_scan_bwd_transforms(q, k, v, logits, gate, A_log, S0, do, dST, dt_bias=dt_bias,
                                     lower_bound=lb, per_channel=per_channel, allow_neg_eigval=neg)
        names = {"gate": "dgate", "logits": "dbeta_logits", "A_log": "dA_log", "dt_bias": "ddt_bias"}
        h = 1e-6
        for name, gname in names.items():
            if x[name] is None:
                continue
            flat = x[name].reshape(-1)
            for i in range(flat.size):
                keep = flat[i]
                flat[i] = keep + h
                lp = loss(x)
                flat[i] = keep - h
                lm = loss(x)
                flat[i] = keep
                fd = (lp - lm) / (2 * h)
                worst = max(worst, abs(fd - gr[gname].reshape(-1)[i]) / max(1.0, abs(fd)))
    return worst


def _tf_no_floor_mask(gate, A_log, dt_bias, logits, ddecay, dbeta, lower_bound, per_channel, neg):
    return _TRUE_TF(gate, A_log, dt_bias, logits, ddecay, dbeta, None, per_channel, neg)


def _tf_softplus_for_sigmoid(gate, A_log, dt_bias, logits, ddecay, dbeta, lower_bound, per_channel,
                             neg):
    out = _TRUE_TF(gate, A_log, dt_bias, logits, ddecay, dbeta, lower_bound, per_channel, neg)
    x = gate + (0.0 if dt_bias is None else dt_bias)
    s = 1 / (1 + np.exp(-x))
    out["dgate"] = out["dgate"] / np.where(s == 0, 1, s) * np.log1p(np.exp(x))
    return out


def _tf_no_eigval_factor(gate, A_log, dt_bias, logits, ddecay, dbeta, lower_bound, per_channel, neg):
    return _TRUE_TF(gate, A_log, dt_bias, logits, ddecay, dbeta, lower_bound, per_channel, False)


def _tf_dA_without_exp(gate, A_log, dt_bias, logits, ddecay, dbeta, lower_bound, per_channel, neg):
    out = _TRUE_TF(gate, A_log, dt_bias, logits, ddecay, dbeta, lower_bound, per_channel, neg)
    out["dA_log"] = out["dA_log"] * np.exp(-A_log)
    return out


TF_MUTANTS = [_tf_no_floor_mask, _tf_softplus_for_sigmoid, _tf_no_eigval_factor, _tf_dA_without_exp]


def test_transform_backward_pin():
    err = pin_transform_finite_differences()
    print(f"pin_transform_finite_differences: {err:.2e}")
    assert err < 1e-7


@pytest.mark.parametrize("mutant", TF_MUTANTS, ids=lambda m: m.__name__)
def test_transform_backward_pin_catches_planted_mistakes(monkeypatch, mutant):
    monkeypatch.setattr(bwd_mod, "transforms_bwd", mutant)
    assert not pin_transform_finite_differences() < 1e-7
