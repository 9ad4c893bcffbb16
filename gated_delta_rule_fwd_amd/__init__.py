"""MI355X (gfx950) gated delta-rule forward: HIP kernels behind a C ABI.

The library (``libkda.so``, built in-tree by ``gated_delta_rule_fwd_amd.build``)
exports ``kda_fwd_chunked``, ``kda_fwd_chunked_varlen``, ``kda_fwd_chunked_noalloc``,
``kda_fwd_recurrent``, ``kda_decode_step`` and the backward ``kda_bwd``
(declared in ``include/kda.h``); this package binds them for torch tensors.
"""
from .kda import (KdaError, bwd, chunked_workspace_bytes, decode_step, fwd_chunked,  # noqa: F401
                  fwd_chunked_varlen, fwd_recurrent,
                  lib,
                  DECAY_CHANNEL, DECAY_HEAD, DECAY_NONE, KDA_BF16, KDA_F32, LIB_PATH)
