"""GPU parity of the backward (kda_bwd, through the C ABI) against the fp64
backward oracle (oracle.backward.kda_scan_bwd, itself pinned by finite
differences of the forward oracle), every gradient separately: max|err| <=
1e-4 rms(ref) for fp32 activations and 2e-2 rms(ref) for bf16 activations
(the kernels compute in fp32 on the given values)."""

import numpy as np
import pytest
import torch

from gated_delta_rule_fwd_amd import bwd, fwd_chunked
from gated_delta_rule_fwd_amd.inputs import (DECAY_CHANNEL, WORKLOADS, make_inputs,
                                             make_transform_inputs)
from oracle import beta_transform, kda_decay, kda_scan_bwd, kda_scan_bwd_transforms
from oracle.backward import transforms_bwd

from test_gpu_parity import TOL, announce, dev, rel, to_dev

pytestmark = pytest.mark.gpu

CASES = [
    ("fp32_small", {}, {}),
    ("fp32_small", dict(T=37, H=2, DK=64, DV=32, decay="channel_softplus", init_state=True), {}),
    ("fp32_small", dict(T=50, H=1, HV=3, DK=32, DV=64, decay="none", init_state=True),
     dict(softmax_scale=0.37)),
    ("gdn_d128", dict(B=2, T=70, H=2), {}),
    ("gdn_d128", dict(B=1, T=16, H=2, DK=64, DV=128), dict(use_qk_l2norm=False)),
    ("kda_d128", dict(B=1, T=53, H=2, DV=64, init_state=True), {}),
    ("kda_d128", dict(B=1, T=40, H=2, decay="channel_steep"), {}),
    ("gdn_d128", dict(B=1, T=161, H=1, HV=2, init_state=True), {}),
    ("deltanet_d64", dict(B=2, T=33, H=2, HV=4), {}),
    ("deltanet_d64", dict(B=1, T=130, H=2, init_state=True), {}),
    # whole chunks of the backward (32 tokens) and no tail; grouped heads with
    # a per-channel decay
    ("kda_d128", dict(B=1, T=64, H=2, DV=32, init_state=True), {}),
    ("fp32_small", dict(T=45, H=1, HV=2, DK=32, DV=32, decay="channel_softplus", init_state=True), {}),
    ("deltanet_d64", dict(B=1, T=1, H=2, DK=128, DV=32, init_state=True), {}),
    # more 16-column slices than two per CU: the reverse walk takes 32 columns
    # per workgroup (per-head decay and none, bf16 and fp32)
    ("gdn_d128", dict(B=2, T=45, H=36, init_state=True), {}),
    ("deltanet_d64", dict(B=1, T=40, H=72, DK=128, DV=128), {}),
    ("fp32_small", dict(B=1, T=37, H=72, DK=32, DV=128, init_state=True), {}),
    ("gdn_d128", dict(B=1, T=40, H=18, HV=72, init_state=True), {}),
]


@pytest.mark.parametrize("name,kw,args", CASES, ids=lambda x: str(x))
def test_backward_matches_oracle(name, kw, args):
    w = WORKLOADS[name].scaled(**kw)
    announce(f"backward {args} {w}")
    inp = make_inputs(w)
    if not args.get("use_qk_l2norm", True):
        for n in ("q", "k"):
            x = inp[n].double()
            inp[n] = (x / x.norm(dim=-1, keepdim=True)).to(inp[n].dtype)
    g = torch.Generator().manual_seed(5)
    do = torch.randn((w.B, w.T, w.hv, w.DV), generator=g)
    dST = torch.randn((w.B, w.hv, w.DK, w.DV), generator=g)
    d = to_dev(inp)
    out = bwd(d["q"], d["k"], d["v"], d["beta"], d["decay"], d["initial_state"], do.to(dev()),
              dST.to(dev()), **args)
    torch.cuda.synchronize()
    ref = kda_scan_bwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["decay"],
                       inp["initial_state"], do, dST, **args)
    tol = TOL[w.dtype]
    for name_g in ("dq", "dk", "dv", "dbeta", "ddecay", "d_initial_state"):
        if ref[name_g] is None:
            assert out[name_g] is None
            continue
        e = rel(out[name_g], ref[name_g])
        print(f"  {name_g}: err/rms={e:.3e} (tol {tol})", flush=True)
        assert e <= tol, f"{name_g}: {e:.3e} > {tol}"


def test_backward_zero_length_and_no_state_gradients():
    d = dev()
    B, H, D = 1, 2, 32
    q = torch.zeros(B, 0, H, D, device=d)
    beta = torch.zeros(B, 0, H, device=d)
    dST = torch.randn(B, H, D, D, device=d)
    out = bwd(q, q, q, beta, None, None, torch.zeros(B, 0, H, D, device=d), dST)
    torch.cuda.synchronize()
    assert torch.equal(out["d_initial_state"], dST)
    # without a final-state gradient and with do = 0 every gradient is zero
    w = WORKLOADS["gdn_d128"].scaled(B=1, T=20, H=2)
    x = to_dev(make_inputs(w))
    out = bwd(x["q"], x["k"], x["v"], x["beta"], x["decay"], x["initial_state"],
              torch.zeros((1, 20, 2, 128), device=d))
    torch.cuda.synchronize()
    for n, t in out.items():
        assert t is None or float(t.abs().max()) == 0.0, n


# Raw-gate / raw-beta transforms: gradients with respect to the raw inputs
# (oracle.backward.kda_scan_bwd_transforms, pinned by finite differences
# through the transformed forward).
TF_CASES = [
    ("gdn_d128", dict(B=1, T=45, H=2), dict()),
    ("gdn_d128", dict(B=2, T=33, H=2, init_state=True), dict(neg=True, lb=-0.3)),
    ("kda_d128", dict(B=1, T=40, H=2, DV=64), dict(lb=-0.8)),
    ("kda_d128", dict(B=1, T=21, H=2, DV=32), dict(bias=False, neg=True)),
    ("fp32_small", dict(T=37, H=2, decay="channel_softplus", init_state=True), dict(lb=-1.0)),
    ("fp32_small", dict(T=29, H=1, HV=2), dict(sigmoid=False)),
    ("fp32_small", dict(T=29, H=2), dict(gate=False, neg=True)),
]


@pytest.mark.parametrize("name,kw,opts", TF_CASES, ids=lambda x: str(x))
def test_backward_transforms_match_oracle(name, kw, opts):
    w = WORKLOADS[name].scaled(**kw)
    announce(f"backward transforms {opts} {w}")
    raw = make_transform_inputs(w)
    gate_on = opts.get("gate", True)
    sig = opts.get("sigmoid", True)
    neg = opts.get("neg", False)
    lb = opts.get("lb")
    bias = raw["dt_bias"] if opts.get("bias", True) else None
    g = torch.Generator().manual_seed(6)
    do = torch.randn((w.B, w.T, w.hv, w.DV), generator=g)
    dST = torch.randn((w.B, w.hv, w.DK, w.DV), generator=g)
    d = {k: (None if v is None else v.to(dev())) for k, v in raw.items()}
    beta_dev = d["beta_logits"] if sig else d["beta"]
    decay_dev = d["gate"] if gate_on else d["decay"]
    out = bwd(d["q"], d["k"], d["v"], beta_dev, decay_dev, d["initial_state"], do.to(dev()),
              dST.to(dev()), use_gate_in_kernel=gate_on, A_log=d["A_log"] if gate_on else None,
              dt_bias=None if (bias is None or not gate_on) else bias.to(dev()),
              lower_bound=lb if gate_on else None, use_beta_sigmoid_in_kernel=sig,
              allow_neg_eigval=neg)
    torch.cuda.synchronize()
    per_channel = w.decay_kind == DECAY_CHANNEL
    if gate_on and sig:
        ref = kda_scan_bwd_transforms(raw["q"], raw["k"], raw["v"], raw["beta_logits"],
                                      raw["gate"], raw["A_log"], raw["initial_state"], do, dST,
                                      dt_bias=bias, lower_bound=lb, per_channel=per_channel,
                                      allow_neg_eigval=neg)
        pairs = dict(dbeta="dbeta_logits", ddecay="dgate", dA_log="dA_log", ddt_bias="ddt_bias")
    else:
        # one transform alone: the plain backward on the transformed input,
        # and the chain rule of the other from the oracle's transforms_bwd
        logits = raw["beta_logits"].double().numpy()
        beta = beta_transform(logits, neg) if sig else raw["beta"]
        gate = raw["gate"].double().numpy() if gate_on else None
        decay = (kda_decay(gate, raw["A_log"], bias, lb, per_channel=per_channel) if gate_on
                 else raw["decay"])
        ref = kda_scan_bwd(raw["q"], raw["k"], raw["v"], beta, decay, raw["initial_state"], do, dST)
        if gate_on:
            chain = transforms_bwd(gate, raw["A_log"].double().numpy(),
                                   None if bias is None else bias.double().numpy(), logits,
                                   ref["ddecay"], ref["dbeta"], lb, per_channel, neg)
        else:
            # the gate's part of the chain rule on a zero gate, unused
            zero = np.zeros_like(ref["dbeta"])
            chain = transforms_bwd(zero, raw["A_log"].double().numpy(), None, logits, zero,
                                   ref["dbeta"], None, False, neg)
        pairs = {}
        if sig:
            ref["dbeta"] = chain["dbeta_logits"]
        if gate_on:
            ref["ddecay"] = chain["dgate"]
            ref["dA_log"], ref["ddt_bias"] = chain["dA_log"], chain["ddt_bias"]
            pairs = dict(dA_log="dA_log", ddt_bias="ddt_bias")
    tol = TOL[w.dtype]
    for name_g in ("dq", "dk", "dv", "dbeta", "ddecay", "d_initial_state", "dA_log", "ddt_bias"):
        key = pairs.get(name_g, name_g)
        r = ref.get(key)
        if r is None:
            assert out[name_g] is None, name_g
            continue
        e = rel(out[name_g], r)
        print(f"  {name_g}: err/rms={e:.3e} (tol {tol})", flush=True)
        assert e <= tol, f"{name_g}: {e:.3e} > {tol}"
    if lb is not None and gate_on:
        # where the floor is taken the raw gate gets no gradient
        decay = kda_decay(raw["gate"], raw["A_log"], bias, None, per_channel=per_channel)
        floored = torch.from_numpy(np.asarray(decay) < lb)
        assert int(floored.sum()) > 0, "the case takes the floor somewhere"
        assert float(out["ddecay"].cpu()[floored].abs().max()) == 0.0


@pytest.mark.parametrize("name,kw", [
    ("gdn_d128", dict(B=2, T=35, H=2, init_state=True)),
    ("kda_d128", dict(B=1, T=20, H=2, DV=64, init_state=True)),
    ("fp32_small", dict(T=18, H=1, HV=2, DK=64, DV=32, init_state=True)),
], ids=lambda x: str(x))
def test_backward_value_major_states(name, kw):
    """state_v_first: the initial state, its gradient and the final-state
    gradient are [B, HV, DV, DK]; every gradient equals the key-major one's
    (the same oracle, the states transposed)."""
    w = WORKLOADS[name].scaled(**kw)
    announce(f"backward value-major {w}")
    inp = make_inputs(w)
    g = torch.Generator().manual_seed(8)
    do = torch.randn((w.B, w.T, w.hv, w.DV), generator=g)
    dST = torch.randn((w.B, w.hv, w.DK, w.DV), generator=g)
    d = to_dev(inp)
    out = bwd(d["q"], d["k"], d["v"], d["beta"], d["decay"],
              d["initial_state"].transpose(-1, -2).contiguous(), do.to(dev()),
              dST.transpose(-1, -2).contiguous().to(dev()), state_v_first=True)
    torch.cuda.synchronize()
    ref = kda_scan_bwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["decay"],
                       inp["initial_state"], do, dST)
    ref["d_initial_state"] = np.swapaxes(ref["d_initial_state"], -1, -2)
    tol = TOL[w.dtype]
    for name_g in ("dq", "dk", "dv", "dbeta", "ddecay", "d_initial_state"):
        if ref[name_g] is None:
            assert out[name_g] is None
            continue
        e = rel(out[name_g], ref[name_g])
        print(f"  {name_g}: err/rms={e:.3e} (tol {tol})", flush=True)
        assert e <= tol, f"{name_g}: {e:.3e} > {tol}"


# Full size: the backward against central differences of the forward (both on
# the GPU), along a random direction per input.  With L = <do, o> +
# <dS_T, S_T>, (L(x + e d) - L(x - e d)) / 2e must equal <grad_x L, d> up to
# O(e^2) and the forward's rounding divided by e.  The workloads' shapes with
# fp32 activations: the fp64 oracle cannot run the whole backward at these
# sizes, and bf16 inputs cannot carry a small step.
FD_EPS = 1e-3
FD_TOL = 1e-2


@pytest.mark.parametrize("name", ["gdn_d128", "kda_d128", "deltanet_d64"])
def test_backward_full_size_directional_derivatives(name):
    w = WORKLOADS[name].scaled(dtype="f32")
    announce(f"backward directional derivatives at full size {w}")
    d = to_dev(make_inputs(w))
    g = torch.Generator(device=dev()).manual_seed(11)
    do = torch.randn((w.B, w.T, w.hv, w.DV), device=dev(), generator=g)
    dST = torch.randn((w.B, w.hv, w.DK, w.DV), device=dev(), generator=g)
    grads = bwd(d["q"], d["k"], d["v"], d["beta"], d["decay"], d["initial_state"], do, dST)

    def loss(x):
        o, st = fwd_chunked(x["q"], x["k"], x["v"], x["beta"], x["decay"], x["initial_state"],
                            chunk_size=w.chunk)
        return float((o.double() * do.double()).sum() + (st.double() * dST.double()).sum())

    names = [("q", "dq"), ("k", "dk"), ("v", "dv"), ("beta", "dbeta")]
    if d["decay"] is not None:
        names.append(("decay", "ddecay"))
    if d["initial_state"] is not None:
        names.append(("initial_state", "d_initial_state"))
    for x_name, g_name in names:
        delta = torch.randn(d[x_name].shape, device=dev(), generator=g)
        if x_name in ("beta", "decay"):
            delta = delta * d[x_name]          # relative steps: beta stays in (0, 1), the decay <= 0
        plus, minus = dict(d), dict(d)
        plus[x_name] = d[x_name] + FD_EPS * delta
        minus[x_name] = d[x_name] - FD_EPS * delta
        fd = (loss(plus) - loss(minus)) / (2 * FD_EPS)
        an = float((grads[g_name].double() * delta.double()).sum())
        err = abs(fd - an) / max(abs(an), 1e-30)
        print(f"  {g_name}: analytic {an:.6e} difference quotient {fd:.6e} rel {err:.2e}", flush=True)
        assert err <= FD_TOL, f"{g_name}: {err:.2e} > {FD_TOL}"
