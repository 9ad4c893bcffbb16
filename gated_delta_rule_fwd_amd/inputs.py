"""Seeded synthetic inputs for the gated delta-rule forward.

This module draws random tensors and nothing else: it holds none of the
method's arithmetic, so the CPU oracle and the HIP path can both be fed from
it.  Draws use NumPy's PCG64 ``default_rng(seed)`` in a fixed order (q, k, v,
beta logits, decay source, initial state), in float32, and are rounded to the
activation dtype with torch's round-to-nearest-even cast.  The tensors that
come back are CPU tensors holding exactly the values a kernel receives.

Workloads (the value distributions of the five standard cases):

* ``fp32_small``   fp32, B1 T64 H2 D32, chunk 16, decay -0.01|N(0,1)| per
  (token, head), zero initial state;
* ``deltanet_d64`` bf16, B4 T2048 H16 D64, chunk 64, no decay;
* ``gdn_d128``     bf16, B8 T4096 H16 D128, chunk 64, decay log(sigmoid(N(2,1)))
  per (token, head), initial state 0.1 N(0,1);
* ``kda_d128``     bf16, B2 T8192 H32 D128, chunk 64, per-key-channel decay
  -softplus(N(-3,1)), zero initial state;
* ``decode_d128``  bf16, B256 H32 D128, one token, decay log(sigmoid(N(2,1)))
  per (batch, head), state 0.1 N(0,1) updated in place.

q, k, v are N(0,1) and are passed raw with ``use_qk_l2norm`` on; beta is
sigmoid(N(0,1)).

``make_transform_inputs`` draws the raw inputs of the in-kernel transforms
instead: a raw gate N(0,1) in the decay's shape, A_log 0.3 N(0,1) per head
(near zero), dt_bias U(-2, 0) per head (or per head and key channel) and beta
logits N(0,1).
"""

from __future__ import annotations

import dataclasses

import numpy as np
import torch

DECAY_NONE, DECAY_HEAD, DECAY_CHANNEL = 0, 1, 2


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str            # "f32" | "bf16"
    B: int
    T: int                # tokens per sequence (1 for decode)
    H: int
    DK: int
    DV: int
    chunk: int            # 0 for decode
    decay: str            # "none" | "head_small" | "head_logsig" | "channel_softplus"
                          # | "channel_strong" | "channel_steep" | "channel_extreme"
                          # | "channel_mild_edge" | "channel_mixed"
    init_state: bool
    decode: bool = False
    seed: int = 1000
    HV: int = 0           # value (recurrent) heads, a multiple of H; 0 means H

    @property
    def hv(self) -> int:
        return self.HV or self.H

    @property
    def decay_kind(self) -> int:
        return {"none": DECAY_NONE, "channel_softplus": DECAY_CHANNEL,
                "channel_strong": DECAY_CHANNEL, "channel_steep": DECAY_CHANNEL,
                "channel_extreme": DECAY_CHANNEL, "channel_mild_edge": DECAY_CHANNEL,
                "channel_mixed": DECAY_CHANNEL}.get(self.decay, DECAY_HEAD)

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "fp32_small": Workload("fp32_small", "f32", 1, 64, 2, 32, 32, 16, "head_small", False, seed=1000),
    "deltanet_d64": Workload("deltanet_d64", "bf16", 4, 2048, 16, 64, 64, 64, "none", False, seed=1001),
    "gdn_d128": Workload("gdn_d128", "bf16", 8, 4096, 16, 128, 128, 64, "head_logsig", True, seed=1002),
    "kda_d128": Workload("kda_d128", "bf16", 2, 8192, 32, 128, 128, 64, "channel_softplus", False, seed=1003),
    "decode_d128": Workload("decode_d128", "bf16", 256, 1, 32, 128, 128, 0, "head_logsig", True,
                            decode=True, seed=1004),
}


def torch_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def _softplus(x):
    return np.logaddexp(0.0, x)


def make_inputs(w: Workload, seed: int | None = None) -> dict:
    """Draw one batch of inputs for workload ``w``.

    Returns a dict of CPU tensors: q, k [B,T,H,DK] (decode: [B,H,DK]),
    v [B,T,HV,DV], beta [B,T,HV], decay (None, [B,T,HV] or [B,T,HV,DK]) in the
    activation dtype, and initial_state [B,HV,DK,DV] fp32 or None (HV = H
    unless the workload sets more value heads).
    """
    rng = np.random.default_rng(w.seed if seed is None else seed)
    dt = torch_dtype(w.dtype)
    qk_lead = (w.B, w.H) if w.decode else (w.B, w.T, w.H)
    lead = (w.B, w.hv) if w.decode else (w.B, w.T, w.hv)

    def normal(shape):
        return rng.standard_normal(shape, dtype=np.float32)

    def act(x):
        return torch.from_numpy(np.ascontiguousarray(x)).to(dt)

    q = act(normal(qk_lead + (w.DK,)))
    k = act(normal(qk_lead + (w.DK,)))
    v = act(normal(lead + (w.DV,)))
    beta = act(1.0 / (1.0 + np.exp(-normal(lead))))
    if w.decay == "none":
        decay = None
    elif w.decay == "head_small":
        decay = act(-0.01 * np.abs(normal(lead)))
    elif w.decay == "head_logsig":
        # log(sigmoid(x)) = -softplus(-x), x ~ N(2, 1)
        decay = act(-_softplus(-(2.0 + normal(lead))))
    elif w.decay == "channel_softplus":
        decay = act(-_softplus(-3.0 + normal(lead + (w.DK,))))
    elif w.decay == "channel_strong":
        # a 16-token block decays by exp(-6) to exp(-14) in most channels
        decay = act(-_softplus(-1.0 + normal(lead + (w.DK,))))
    elif w.decay == "channel_steep":
        # strong per-channel decay: a 16-token block decays by about exp(-20)
        # in most channels, still far from fp32 underflow
        decay = act(-_softplus(1.0 + normal(lead + (w.DK,))))
    elif w.decay == "channel_extreme":
        # about -10 per token: a 16-token block decays by about exp(-160)
        decay = act(-_softplus(10.0 + 2.0 * normal(lead + (w.DK,))))
    elif w.decay == "channel_mild_edge":
        # -0.66 .. -0.74 per token: every 4 tokens decay by just under exp(-3)
        # in every channel, half blocks by nearly exp(-6)
        decay = act(-rng.uniform(0.66, 0.74, lead + (w.DK,)).astype(np.float32))
    elif w.decay == "channel_mixed":
        # spans of 96 tokens alternate between the workload's decay and a
        # steep one, so chunks of either kind, and chunks holding both, follow
        # one another in one sequence
        mild = -_softplus(-3.0 + normal(lead + (w.DK,)))
        steep = -_softplus(1.0 + normal(lead + (w.DK,)))
        t_idx = np.arange(w.T).reshape((1, w.T) + (1,) * (len(lead) - 2))
        decay = act(np.where(((t_idx // 96) % 2 == 1)[..., None], steep, mild))
    else:
        raise ValueError(w.decay)
    init = None
    if w.init_state:
        init = torch.from_numpy(0.1 * normal((w.B, w.hv, w.DK, w.DV)))
    return dict(q=q, k=k, v=v, beta=beta, decay=decay, initial_state=init)


def make_transform_inputs(w: Workload, seed: int | None = None) -> dict:
    """Inputs for the raw-gate / raw-beta transforms of workload ``w``.

    Everything ``make_inputs(w, seed)`` returns, and from a second stream gate (None, [lead] or [lead, DK] as w's decay kind, in
    the activation dtype), beta_logits [lead] (activation dtype), A_log [H]
    and dt_bias [H] or [H, DK] (fp32).
    """
    base = make_inputs(w, seed)
    rng = np.random.default_rng((w.seed if seed is None else seed) + 7919)
    dt = torch_dtype(w.dtype)
    lead = (w.B, w.hv) if w.decode else (w.B, w.T, w.hv)

    def act(x):
        return torch.from_numpy(np.ascontiguousarray(x)).to(dt)

    kind = w.decay_kind
    gshape = lead + ((w.DK,) if kind == DECAY_CHANNEL else ())
    bshape = (w.hv, w.DK) if kind == DECAY_CHANNEL else (w.hv,)
    gate = act(rng.standard_normal(gshape, dtype=np.float32)) if kind != DECAY_NONE else None
    beta_logits = act(rng.standard_normal(lead, dtype=np.float32))
    A_log = torch.from_numpy(0.3 * rng.standard_normal((w.hv,), dtype=np.float32))
    dt_bias = torch.from_numpy(rng.uniform(-2.0, 0.0, bshape).astype(np.float32))
    return dict(base, gate=gate, beta_logits=beta_logits, A_log=A_log, dt_bias=dt_bias)
