"""The allocation-free chunked entry point (kda_fwd_chunked_noalloc) against
kda_fwd_chunked with a caller workspace, through the C ABI: two calls in a
row on the shared per-device scratch, the second with a smaller input (so it
runs over what the first left there), each bitwise equal to the workspace
call and within the bf16 bar of the oracle.  A third call is longer than the
scratch holds in one pass (several segments of chunks)."""

import numpy as np
import pytest
import torch

from gated_delta_rule_fwd_amd import fwd_chunked
from gated_delta_rule_fwd_amd.inputs import WORKLOADS, make_inputs
from gated_delta_rule_fwd_amd.kda import NOALLOC_WORKSPACE_BYTES, chunked_workspace_bytes, \
    fwd_chunked_noalloc
from oracle import kda_scan

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


def _rel(out, ref):
    out = out.detach().double().cpu().numpy()
    return float(np.abs(out - ref).max() / np.sqrt(np.mean(ref * ref)))


def _case(w, with_oracle=True):
    print(f"\n[case] noalloc {w}", flush=True)
    dev = torch.device("cuda:0")
    inp = make_inputs(w)
    d = {k: (None if v is None else v.to(dev)) for k, v in inp.items()}
    args = (d["q"], d["k"], d["v"], d["beta"], d["decay"], d["initial_state"])
    o1, S1 = fwd_chunked_noalloc(*args, chunk_size=w.chunk)
    o2, S2 = fwd_chunked(*args, chunk_size=w.chunk)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2), "noalloc differs from the workspace call"
    if with_oracle:
        o_ref, S_ref = kda_scan(inp["q"], inp["k"], inp["v"], inp["beta"], inp["decay"],
                                inp["initial_state"])
        eo, es = _rel(o1, o_ref), _rel(S1, S_ref)
        print(f"  noalloc: o err/rms={eo:.3e} state err/rms={es:.3e}", flush=True)
        assert eo <= TOL[w.dtype] and es <= TOL[w.dtype]


def test_noalloc_two_calls_second_smaller():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _case(WORKLOADS["kda_d128"].scaled(B=2, T=300, H=4, init_state=True))
    _case(WORKLOADS["kda_d128"].scaled(B=1, T=130, H=2))
    _case(WORKLOADS["gdn_d128"].scaled(B=2, T=200, H=4, init_state=True))
    _case(WORKLOADS["gdn_d128"].scaled(B=1, T=70, H=2, chunk=32))


def test_noalloc_longer_than_the_scratch():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    # kda_d128 at full size: 549 MB of records, several segments through 64 MiB
    w = WORKLOADS["kda_d128"]
    assert chunked_workspace_bytes(w.B, w.T, w.H, w.H, w.DK, w.DV, torch.bfloat16,
                                   w.decay_kind, w.chunk) > 4 * NOALLOC_WORKSPACE_BYTES
    _case(w, with_oracle=False)
