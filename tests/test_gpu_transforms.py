"""GPU parity of the in-kernel input transforms (raw gate, floor, raw beta).

Each case runs an entry point with the raw inputs and the transform flags,
and compares it with the fp64 oracle fed the oracle's own transforms of the
same raw values (oracle.transforms: ejkernel kda_decay; TileOPs GDNFwdOp /
KDAFwdOp use_gate_in_kernel, lower_bound, use_beta_sigmoid_in_kernel,
allow_neg_eigval).  Bar as for the untransformed paths: max|err| <=
1e-4 * rms for fp32 activations, 2e-2 * rms for bf16.
"""

import sys

import numpy as np
import pytest
import torch

from gated_delta_rule_fwd_amd import decode_step, fwd_chunked, fwd_chunked_varlen, fwd_recurrent
from gated_delta_rule_fwd_amd.inputs import DECAY_CHANNEL, WORKLOADS, make_transform_inputs
from oracle import beta_transform, kda_decay, kda_scan

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def rel(out, ref):
    out = out.detach().double().cpu().numpy()
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.abs(out - ref).max() / max(np.sqrt(np.mean(ref * ref)), 1e-30))


def check(name, o, S, o_ref, S_ref, tol):
    eo, es = rel(o, o_ref), rel(S, S_ref)
    print(f"  {name}: o err/rms={eo:.3e}  state err/rms={es:.3e}  (tol {tol})", flush=True)
    assert eo <= tol and es <= tol


def prepare(w, opts):
    """(device kwargs for the binding, device tensors, oracle decay, oracle beta)."""
    raw = make_transform_inputs(w)
    d = {k: (None if v is None else v.to(dev())) for k, v in raw.items()}
    gate_on = opts.get("gate", True) and w.decay != "none"
    sig = opts.get("sigmoid", True)
    neg = opts.get("neg", False)
    lb = opts.get("lb")
    bias = opts.get("bias", True)
    if gate_on:
        decay_dev = d["gate"]
        decay_ref = kda_decay(raw["gate"], raw["A_log"], raw["dt_bias"] if bias else None, lb,
                              per_channel=w.decay_kind == DECAY_CHANNEL)
    else:
        decay_dev, decay_ref = d["decay"], raw["decay"]
    beta_dev = d["beta_logits"] if sig else d["beta"]
    beta_ref = beta_transform(raw["beta_logits"], neg) if sig else raw["beta"]
    kw = dict(use_gate_in_kernel=gate_on, A_log=d["A_log"] if gate_on else None,
              dt_bias=d["dt_bias"] if (gate_on and bias) else None,
              lower_bound=lb if gate_on else None,
              use_beta_sigmoid_in_kernel=sig, allow_neg_eigval=neg)
    return kw, d, raw, decay_dev, beta_dev, decay_ref, beta_ref


CHUNK_CASES = [
    ("gdn_d128", dict(B=1, T=150, H=4), {}),
    ("gdn_d128", dict(B=2, T=70, H=64), dict(neg=True)),
    ("gdn_d128", dict(B=1, T=90, H=2, chunk=32), dict(bias=False, lb=-0.5)),
    ("kda_d128", dict(B=1, T=130, H=2, init_state=True), dict(lb=-0.8, neg=True)),
    ("kda_d128", dict(B=1, T=100, H=2, chunk=32), dict(sigmoid=False)),
    ("kda_d128", dict(B=1, T=70, H=2, chunk=16), dict(gate=False)),
    ("fp32_small", dict(T=70, chunk=32, decay="channel_softplus"), dict(lb=-1.0)),
    ("fp32_small", dict(T=45, H=3), dict(neg=True)),
    ("deltanet_d64", dict(B=1, T=100, H=4), dict(neg=True)),
]


@pytest.mark.parametrize("name,kw,opts", CHUNK_CASES, ids=lambda x: str(x))
def test_chunked_transforms(name, kw, opts):
    w = WORKLOADS[name].scaled(**kw)
    print(f"\n[case] chunked transforms {opts} {w}", flush=True)
    tkw, d, raw, decay_dev, beta_dev, decay_ref, beta_ref = prepare(w, opts)
    o, S = fwd_chunked(d["q"], d["k"], d["v"], beta_dev, decay_dev, d["initial_state"],
                       chunk_size=w.chunk, **tkw)
    torch.cuda.synchronize()
    o_ref, S_ref = kda_scan(raw["q"], raw["k"], raw["v"], beta_ref, decay_ref,
                            raw["initial_state"])
    check("chunked", o, S, o_ref, S_ref, TOL[w.dtype])


def test_varlen_transforms():
    lens = [70, 0, 130, 33]
    w = WORKLOADS["kda_d128"].scaled(B=1, T=sum(lens), H=2)
    opts = dict(lb=-5.0)
    print(f"\n[case] varlen transforms {lens} {opts} {w}", flush=True)
    tkw, d, raw, decay_dev, beta_dev, decay_ref, beta_ref = prepare(w, opts)
    cu = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32)
    o, S = fwd_chunked_varlen(d["q"], d["k"], d["v"], beta_dev, cu, decay=decay_dev,
                              chunk_size=w.chunk, **tkw)
    torch.cuda.synchronize()
    o_ref = np.zeros((1, w.T, w.H, w.DV))
    S_ref = np.zeros((len(lens), w.H, w.DK, w.DV))
    for n in range(len(lens)):
        a, b = int(cu[n]), int(cu[n + 1])
        o_n, S_n = kda_scan(raw["q"][:, a:b], raw["k"][:, a:b], raw["v"][:, a:b],
                            beta_ref[:, a:b], decay_ref[:, a:b])
        o_ref[:, a:b] = o_n
        S_ref[n] = S_n[0]
    check("varlen", o, S, o_ref, S_ref, TOL[w.dtype])


REC_CASES = [
    ("gdn_d128", dict(B=2, T=40, H=3), dict(neg=True)),
    ("kda_d128", dict(B=1, T=33, H=2), dict(lb=-1.0)),
    ("fp32_small", dict(T=37, decay="channel_softplus", init_state=True, DK=64, DV=32),
     dict(bias=False)),
]


@pytest.mark.parametrize("name,kw,opts", REC_CASES, ids=lambda x: str(x))
def test_recurrent_transforms(name, kw, opts):
    w = WORKLOADS[name].scaled(**kw)
    print(f"\n[case] recurrent transforms {opts} {w}", flush=True)
    tkw, d, raw, decay_dev, beta_dev, decay_ref, beta_ref = prepare(w, opts)
    o, S = fwd_recurrent(d["q"], d["k"], d["v"], beta_dev, decay_dev, d["initial_state"], **tkw)
    torch.cuda.synchronize()
    o_ref, S_ref = kda_scan(raw["q"], raw["k"], raw["v"], beta_ref, decay_ref,
                            raw["initial_state"])
    check("recurrent", o, S, o_ref, S_ref, TOL[w.dtype])


DEC_CASES = [
    (dict(B=4, H=8), dict(neg=True)),
    (dict(B=3, H=5, decay="channel_softplus"), dict(lb=-0.3)),
    (dict(B=2, H=3, dtype="f32"), dict(bias=False)),
]


@pytest.mark.parametrize("kw,opts", DEC_CASES, ids=lambda x: str(x))
def test_decode_transforms(kw, opts):
    w = WORKLOADS["decode_d128"].scaled(**kw)
    print(f"\n[case] decode transforms {opts} {w}", flush=True)
    tkw, d, raw, decay_dev, beta_dev, decay_ref, beta_ref = prepare(w, opts)
    state = d["initial_state"].clone()
    o = decode_step(d["q"], d["k"], d["v"], beta_dev, decay_dev, state, **tkw)
    torch.cuda.synchronize()
    o_ref, S_ref = kda_scan(raw["q"][:, None], raw["k"][:, None], raw["v"][:, None],
                            beta_ref[:, None], decay_ref[:, None], raw["initial_state"])
    check("decode", o, state, o_ref[:, 0], S_ref, TOL[w.dtype])


def test_transforms_off_is_bitwise_the_plain_call():
    # with every flag off the entry point reads decay and beta as given
    w = WORKLOADS["gdn_d128"].scaled(B=1, T=130, H=4)
    print(f"\n[case] transforms off {w}", flush=True)
    raw = make_transform_inputs(w)
    d = {k: (None if v is None else v.to(dev())) for k, v in raw.items()}
    a = fwd_chunked(d["q"], d["k"], d["v"], d["beta"], d["decay"], d["initial_state"])
    b = fwd_chunked(d["q"], d["k"], d["v"], d["beta"], d["decay"], d["initial_state"],
                    A_log=d["A_log"], dt_bias=d["dt_bias"])
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_full_size_raw_gate_kda_every_head():
    # kda_d128 at its full size from the raw gate and raw beta, in the
    # configuration of the benchmark's raw-gate extra (floor -5, sigmoid);
    # the oracle transforms and scans every (b, h) over the whole sequence
    w = WORKLOADS["kda_d128"]
    print(f"\n[case] raw gate full size {w}", flush=True)
    raw = make_transform_inputs(w)
    d = {k: (None if v is None else v.to(dev())) for k, v in raw.items()}
    o, S = fwd_chunked(d["q"], d["k"], d["v"], d["beta_logits"], d["gate"], d["initial_state"],
                       chunk_size=w.chunk, use_gate_in_kernel=True, A_log=d["A_log"],
                       dt_bias=d["dt_bias"], lower_bound=-5.0, use_beta_sigmoid_in_kernel=True)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(S).all()
    o, S = o.cpu(), S.cpu()
    del d
    torch.cuda.empty_cache()
    o_ref, S_ref = [], []
    for b in range(w.B):
        sl = slice(b, b + 1)
        dec = kda_decay(raw["gate"][sl], raw["A_log"], raw["dt_bias"], -5.0, per_channel=True)
        o_b, S_b = kda_scan(raw["q"][sl], raw["k"][sl], raw["v"][sl],
                            beta_transform(raw["beta_logits"][sl]), dec, None)
        o_ref.append(o_b)
        S_ref.append(S_b)
    check("raw gate every head", o, S, np.concatenate(o_ref), np.concatenate(S_ref), TOL[w.dtype])
