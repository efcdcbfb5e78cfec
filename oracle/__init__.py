"""CPU oracle for the bucketed classifier-free guidance (BCG) guided denoising step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or run
anything in this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (no kernels, headers, helpers, tables or constant generators); both
sides are fed the same seeded inputs from ``workloads``.

Two modes:

* ``definition`` (mode D): the method written out plainly in float64, one
  function per step of the path, each citing the passage it follows.  This is
  the oracle proper.
* ``mirror32`` (mode M): the same steps evaluated as a fixed sequence of
  IEEE float32 operations (no fused multiply-add, correctly rounded division).
  It exists because bf16 storage turns float32 results into 8-bit-significand
  codes: a final-latent bound of 2e-2 is below one bf16 ulp for |x| >= 4, so
  the code chosen must be decided in the same precision and order as the
  kernel does it.  Mode M is itself pinned to mode D (per-step tolerance) and
  to the special cases the pages fix.

A third module, ``weight_patch``, is the oracle of the weight-patch workload
(a weight with its diff and low-rank patches applied, stored with stochastic
rounding): float64 definition, the kernel's float32 order and the
counter-based generator of the rounding bits.

Parity status per function is stated in each module's header.
"""
from . import definition, mirror32, weight_patch  # noqa: F401
