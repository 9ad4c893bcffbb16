"""CPU oracle for the gated delta-rule forward and backward (fp64, NumPy).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it; the library and its Python
binding never import it, and it imports nothing from them.

* ``scan.kda_scan`` -- the oracle: the sequential recurrence, token by token.
* ``scan.kda_decode`` -- the single-step mode (the scan with T = 1).
* ``transforms.kda_decay`` / ``transforms.beta_transform`` -- the optional
  raw-gate and raw-beta input transforms, in fp64.
* ``backward.kda_scan_bwd`` -- the gradients of the scan with respect to
  every input, by a hand-written reverse pass over the tokens;
  ``kda_scan_bwd_transforms`` carries them through the raw-gate and raw-beta
  transforms.
* ``chunked_ref.kda_chunked_ref`` -- the chunked WY form, kept only to pin the
  chunk algebra against the scan on the CPU; it is not used as a reference for
  the GPU path.
"""
from .scan import kda_scan, kda_decode, kda_scan_heads, resolve_scale, l2_normalize  # noqa: F401
from .chunked_ref import kda_chunked_ref  # noqa: F401
from .transforms import beta_transform, kda_decay, softplus  # noqa: F401
from .backward import kda_scan_bwd, kda_scan_bwd_transforms  # noqa: F401
