"""GPU parity for the boundary arguments that shape the query and key rows:
use_qk_l2norm off (with rows normalised by the caller), an explicit
softmax_scale, a zero or NaN scale (the default DK^-0.5), and all-zero q and
k rows under the in-kernel L2 norm (divided by the 1e-12 floor, so they stay
zero).  Every entry point (chunked, packed varlen, recurrent, decode) against
the fp64 oracle fed the same values and the same arguments.

ejkernel kda parameter list: softmax_scale (None means the inverse square
root of the head size) and use_qk_l2norm; TileOPs GLA ops: a non-positive
scale selects the default.
"""

import math

import numpy as np
import pytest
import torch

from gated_delta_rule_fwd_amd import decode_step, fwd_chunked, fwd_chunked_varlen, fwd_recurrent
from gated_delta_rule_fwd_amd.inputs import WORKLOADS, make_inputs, torch_dtype
from oracle import kda_decode, kda_scan

from test_gpu_parity import TOL, announce, check, dev, to_dev

pytestmark = pytest.mark.gpu

CASES = ["l2_off", "scale_0.37", "scale_0", "scale_nan", "zero_rows"]

WORKLOADS_SMALL = [
    # bf16 with the raw-row state kernel (per-head decay, chunk 64)
    ("gdn_d128", dict(B=1, T=150, H=2, init_state=True)),
    # bf16 per-channel decay
    ("kda_d128", dict(B=1, T=130, H=2)),
    # bf16 without decay, DK = DV = 64, chunk 32
    ("deltanet_d64", dict(B=2, T=100, H=2, chunk=32)),
    # fp32 activations
    ("fp32_small", dict(T=70, H=2)),
]


def _unit_rows(x, dt):
    """rows normalised in fp64 by the caller, then cast to the activation dtype"""
    x = x.double()
    return (x / x.norm(dim=-1, keepdim=True)).to(dt)


def apply_case(inp, case, dt, decode=False):
    """Modify the inputs for the case in place; return the keyword arguments
    both the library and the oracle get."""
    if case == "l2_off":
        inp["q"] = _unit_rows(inp["q"], dt)
        inp["k"] = _unit_rows(inp["k"], dt)
        return dict(use_qk_l2norm=False)
    if case == "scale_0.37":
        return dict(softmax_scale=0.37)
    if case == "scale_0":
        return dict(softmax_scale=0.0)
    if case == "scale_nan":
        return dict(softmax_scale=math.nan)
    if case == "zero_rows":
        if decode:
            inp["q"][1, 0] = 0
            inp["k"][0, 1] = 0
        else:
            T = inp["q"].shape[1]
            inp["q"][0, min(5, T - 1), 0] = 0
            inp["k"][0, min(9, T - 1), inp["k"].shape[2] - 1] = 0
            inp["k"][0, T - 1, 0] = 0          # the last token of the sequence
        return {}
    raise ValueError(case)


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("name,kw", WORKLOADS_SMALL, ids=lambda x: str(x))
def test_chunked_and_recurrent_boundary_args(name, kw, case):
    w = WORKLOADS[name].scaled(**kw)
    announce(f"boundary args {case} chunked + recurrent {w}")
    inp = make_inputs(w)
    args = apply_case(inp, case, torch_dtype(w.dtype))
    d = to_dev(inp)
    x = (d["q"], d["k"], d["v"], d["beta"], d["decay"], d["initial_state"])
    o_c, S_c = fwd_chunked(*x, chunk_size=w.chunk, **args)
    o_r, S_r = fwd_recurrent(*x, **args)
    torch.cuda.synchronize()
    o_ref, S_ref = kda_scan(inp["q"], inp["k"], inp["v"], inp["beta"], inp["decay"],
                            inp["initial_state"], **args)
    assert np.isfinite(o_ref).all()
    check(f"chunked {case}", o_c, S_c, o_ref, S_ref, TOL[w.dtype])
    check(f"recurrent {case}", o_r, S_r, o_ref, S_ref, TOL[w.dtype])
    if case == "zero_rows":
        # a zero query reads nothing at its token
        t = min(5, w.T - 1)
        assert float(o_c[0, t, 0].abs().max()) == 0.0 and float(o_r[0, t, 0].abs().max()) == 0.0


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("name", ["gdn_d128", "kda_d128", "fp32_small"])
def test_varlen_boundary_args(name, case):
    lens = [70, 0, 65, 17]
    T = sum(lens)
    w = WORKLOADS[name].scaled(B=1, T=T, H=2, init_state=False)
    announce(f"boundary args {case} varlen {lens} {w}")
    inp = make_inputs(w)
    args = apply_case(inp, case, torch_dtype(w.dtype))
    d = to_dev(inp)
    cu = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32)
    o, S = fwd_chunked_varlen(d["q"], d["k"], d["v"], d["beta"], cu, decay=d["decay"],
                              chunk_size=w.chunk, **args)
    torch.cuda.synchronize()
    o_ref = np.zeros((1, T, w.H, w.DV))
    S_ref = np.zeros((len(lens), w.H, w.DK, w.DV))
    for n in range(len(lens)):
        a, b = int(cu[n]), int(cu[n + 1])
        sl = lambda x: None if x is None else x[:, a:b]
        o_n, S_n = kda_scan(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), sl(inp["beta"]),
                            sl(inp["decay"]), None, **args)
        o_ref[:, a:b] = o_n
        S_ref[n] = S_n[0]
    check(f"varlen {case}", o, S, o_ref, S_ref, TOL[w.dtype])


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("kw", [dict(B=3, H=4), dict(B=2, H=3, decay="channel_softplus"),
                                dict(B=2, H=2, DK=64, DV=32, decay="none"),
                                dict(B=2, H=3, dtype="f32")], ids=lambda x: str(x))
def test_decode_boundary_args(kw, case):
    w = WORKLOADS["decode_d128"].scaled(**kw)
    announce(f"boundary args {case} decode {w}")
    inp = make_inputs(w)
    args = apply_case(inp, case, torch_dtype(w.dtype), decode=True)
    d = to_dev(inp)
    state = d["initial_state"].clone()
    o = decode_step(d["q"], d["k"], d["v"], d["beta"], d["decay"], state, **args)
    torch.cuda.synchronize()
    o_ref, S_ref = kda_decode(inp["q"], inp["k"], inp["v"], inp["beta"], inp["decay"],
                              inp["initial_state"], **args)
    check(f"decode {case}", o, state, o_ref, S_ref, TOL[w.dtype])
