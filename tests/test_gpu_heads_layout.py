"""GPU parity for grouped value heads (HV a multiple of H) and the
value-major state layout (TileOPs GDNFwdOp / KDAFwdOp: HV recurrent heads,
``state_v_first``), on every entry point.

The oracle scan takes q, k with H heads and v with HV heads (value head hv
reads q/k head hv // (HV // H)); a value-major state is the oracle's
key-major state with its last two axes swapped.  Bar as elsewhere:
max|err| <= 1e-4 * rms for fp32 activations, 2e-2 * rms for bf16.
"""

import numpy as np
import pytest
import torch

from gated_delta_rule_fwd_amd import decode_step, fwd_chunked, fwd_chunked_varlen, fwd_recurrent
from gated_delta_rule_fwd_amd.inputs import DECAY_CHANNEL, WORKLOADS, make_inputs, \
    make_transform_inputs
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


def vm(x):
    """key-major state [.., DK, DV] <-> value-major [.., DV, DK]"""
    if x is None:
        return None
    if isinstance(x, np.ndarray):
        return np.ascontiguousarray(np.swapaxes(x, -1, -2))
    return x.transpose(-1, -2).contiguous()


def to_dev(inp):
    return {k: (None if v is None else v.to(dev())) for k, v in inp.items()}


CHUNK_CASES = [
    ("gdn_d128", dict(B=1, T=150, H=2, HV=4, init_state=True), False),
    ("gdn_d128", dict(B=2, T=70, H=8, HV=32), False),          # 32 value heads: narrower slices
    ("kda_d128", dict(B=1, T=100, H=1, HV=3, chunk=32), False),
    ("deltanet_d64", dict(B=1, T=70, H=2, HV=8), False),
    ("gdn_d128", dict(B=1, T=130, H=4, init_state=True), True),
    ("kda_d128", dict(B=1, T=90, H=1, HV=2, init_state=True), True),
    ("fp32_small", dict(T=70, H=1, HV=2, init_state=True, chunk=32), True),
    ("fp32_small", dict(T=45, H=2, HV=6, DK=64, DV=32, decay="channel_softplus"), False),
]


@pytest.mark.parametrize("name,kw,vfirst", CHUNK_CASES, ids=lambda x: str(x))
def test_chunked_heads_and_layout(name, kw, vfirst):
    w = WORKLOADS[name].scaled(**kw)
    print(f"\n[case] chunked heads/layout vfirst={vfirst} {w}", flush=True)
    inp = make_inputs(w)
    d = to_dev(inp)
    init = vm(d["initial_state"]) if vfirst else d["initial_state"]
    o, S = fwd_chunked(d["q"], d["k"], d["v"], d["beta"], d["decay"], init,
                       chunk_size=w.chunk, state_v_first=vfirst)
    torch.cuda.synchronize()
    o_ref, S_ref = kda_scan(inp["q"], inp["k"], inp["v"], inp["beta"], inp["decay"],
                            inp["initial_state"])
    check("chunked", o, S, o_ref, vm(S_ref) if vfirst else S_ref, TOL[w.dtype])


def test_varlen_heads_and_layout():
    lens = [70, 0, 130, 33]
    w = WORKLOADS["gdn_d128"].scaled(B=1, T=sum(lens), H=2, HV=4)
    print(f"\n[case] varlen heads/layout {lens} {w}", flush=True)
    inp = make_inputs(w)
    d = to_dev(inp)
    g = torch.Generator().manual_seed(78)
    s0 = 0.1 * torch.randn((len(lens), w.hv, w.DK, w.DV), generator=g, dtype=torch.float64).float()
    cu = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32)
    o, S = fwd_chunked_varlen(d["q"], d["k"], d["v"], d["beta"], cu, decay=d["decay"],
                              initial_state=vm(s0).to(dev()), chunk_size=w.chunk,
                              state_v_first=True)
    torch.cuda.synchronize()
    o_ref = np.zeros((1, w.T, w.hv, w.DV))
    S_ref = np.zeros((len(lens), w.hv, w.DK, w.DV))
    for n in range(len(lens)):
        a, b = int(cu[n]), int(cu[n + 1])
        o_n, S_n = kda_scan(inp["q"][:, a:b], inp["k"][:, a:b], inp["v"][:, a:b],
                            inp["beta"][:, a:b], inp["decay"][:, a:b], s0[n:n + 1])
        o_ref[:, a:b] = o_n
        S_ref[n] = S_n[0]
    check("varlen", o, S, o_ref, vm(S_ref), TOL[w.dtype])


REC_CASES = [
    ("gdn_d128", dict(B=2, T=40, H=1, HV=3, init_state=True), True),
    ("kda_d128", dict(B=1, T=33, H=2, HV=4), False),
    ("fp32_small", dict(T=37, H=1, HV=2, init_state=True, DK=64, DV=32,
                        decay="channel_softplus"), True),
]


@pytest.mark.parametrize("name,kw,vfirst", REC_CASES, ids=lambda x: str(x))
def test_recurrent_heads_and_layout(name, kw, vfirst):
    w = WORKLOADS[name].scaled(**kw)
    print(f"\n[case] recurrent heads/layout vfirst={vfirst} {w}", flush=True)
    inp = make_inputs(w)
    d = to_dev(inp)
    init = vm(d["initial_state"]) if vfirst else d["initial_state"]
    o, S = fwd_recurrent(d["q"], d["k"], d["v"], d["beta"], d["decay"], init,
                         state_v_first=vfirst)
    torch.cuda.synchronize()
    o_ref, S_ref = kda_scan(inp["q"], inp["k"], inp["v"], inp["beta"], inp["decay"],
                            inp["initial_state"])
    check("recurrent", o, S, o_ref, vm(S_ref) if vfirst else S_ref, TOL[w.dtype])


DEC_CASES = [
    (dict(B=4, H=2, HV=8), False),
    (dict(B=4, H=8), True),
    (dict(B=3, H=1, HV=5, decay="channel_softplus"), True),
    (dict(B=2, H=2, HV=4, DK=64, DV=128), True),
    (dict(B=2, H=3, DK=32, DV=32, decay="none"), True),
    (dict(B=2, H=3, DK=32, DV=128), True),
    (dict(B=2, H=2, DK=128, DV=32), True),
    (dict(B=2, H=1, HV=3, dtype="f32"), True),
]


@pytest.mark.parametrize("kw,vfirst", DEC_CASES, ids=lambda x: str(x))
def test_decode_heads_and_layout(kw, vfirst):
    w = WORKLOADS["decode_d128"].scaled(**kw)
    print(f"\n[case] decode heads/layout vfirst={vfirst} {w}", flush=True)
    inp = make_inputs(w)
    d = to_dev(inp)
    state = vm(d["initial_state"]) if vfirst else d["initial_state"].clone()
    o = decode_step(d["q"], d["k"], d["v"], d["beta"], d["decay"], state, state_v_first=vfirst)
    torch.cuda.synchronize()
    dec = None if inp["decay"] is None else inp["decay"][:, None]
    o_ref, S_ref = kda_scan(inp["q"][:, None], inp["k"][:, None], inp["v"][:, None],
                            inp["beta"][:, None], dec, inp["initial_state"])
    check("decode", o, state, o_ref[:, 0], vm(S_ref) if vfirst else S_ref, TOL[w.dtype])


def test_transforms_with_grouped_heads():
    # A_log and dt_bias are per value head
    w = WORKLOADS["kda_d128"].scaled(B=1, T=100, H=1, HV=2)
    print(f"\n[case] transforms + heads {w}", flush=True)
    raw = make_transform_inputs(w)
    d = to_dev(raw)
    o, S = fwd_chunked(d["q"], d["k"], d["v"], d["beta_logits"], d["gate"], None,
                       use_gate_in_kernel=True, A_log=d["A_log"], dt_bias=d["dt_bias"],
                       lower_bound=-5.0, use_beta_sigmoid_in_kernel=True)
    torch.cuda.synchronize()
    decay = kda_decay(raw["gate"], raw["A_log"], raw["dt_bias"], -5.0,
                      per_channel=w.decay_kind == DECAY_CHANNEL)
    o_ref, S_ref = kda_scan(raw["q"], raw["k"], raw["v"], beta_transform(raw["beta_logits"]),
                            decay)
    check("chunked transforms", o, S, o_ref, S_ref, TOL[w.dtype])


def test_decode_value_major_equals_key_major_bitwise_after_transpose():
    # same arithmetic per element in both layouts is not promised; compare to
    # the oracle's bar, and check the two layouts agree to fp32 rounding
    w = WORKLOADS["decode_d128"].scaled(B=8, H=4)
    print(f"\n[case] decode layouts {w}", flush=True)
    inp = make_inputs(w)
    d = to_dev(inp)
    s_km = d["initial_state"].clone()
    s_vm = vm(d["initial_state"])
    o1 = decode_step(d["q"], d["k"], d["v"], d["beta"], d["decay"], s_km)
    o2 = decode_step(d["q"], d["k"], d["v"], d["beta"], d["decay"], s_vm, state_v_first=True)
    torch.cuda.synchronize()
    assert rel(o2, o1.double().cpu().numpy()) < 1e-5
    assert rel(vm(s_vm), s_km.double().cpu().numpy()) < 1e-5


def test_full_size_grouped_heads_every_head():
    # gdn_d128's shape with 4 q/k heads for its 16 value heads, as the
    # benchmark's grouped-head extra runs it; every (b, value head)
    from test_gpu_parity import full_oracle
    w = WORKLOADS["gdn_d128"].scaled(H=4, HV=16)
    print(f"\n[case] grouped heads full size {w}", flush=True)
    inp = make_inputs(w)
    d = to_dev(inp)
    o, S = fwd_chunked(d["q"], d["k"], d["v"], d["beta"], d["decay"], d["initial_state"],
                       chunk_size=w.chunk)
    torch.cuda.synchronize()
    o_ref, S_ref = full_oracle(inp)
    check("grouped every head", o, S, o_ref, S_ref, TOL[w.dtype])


def test_decode_full_size_value_major():
    # decode_d128 at full size with a value-major state, as the benchmark's
    # value-major extra runs it; every batch entry
    from oracle import kda_decode
    w = WORKLOADS["decode_d128"]
    print(f"\n[case] decode value-major full size {w}", flush=True)
    inp = make_inputs(w)
    d = to_dev(inp)
    state = vm(d["initial_state"])
    o = decode_step(d["q"], d["k"], d["v"], d["beta"], d["decay"], state, state_v_first=True)
    torch.cuda.synchronize()
    o_ref, S_ref = kda_decode(inp["q"], inp["k"], inp["v"], inp["beta"], inp["decay"],
                              inp["initial_state"])
    check("decode value-major every row", o, state, o_ref, vm(S_ref), TOL[w.dtype])
