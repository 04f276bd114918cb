"""Plain fp64 CPU oracle for the hybrid Muon + AdamW optimizer step.

TEST INFRASTRUCTURE ONLY. Nothing in the product package (``muon_adamw_amd``)
imports, calls or links anything here; only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may use
it. It shares no code with the HIP path: the only thing both sides consume is
the seeded input generator in ``workloads``, which holds no optimizer
arithmetic.

Every function is written from the pages' update rules, in their order and
notation, in float64 with numpy (a matrix product is the only library
primitive used):

* ``muon``  -- momentum EMA, Nesterov lerp, Frobenius normalisation, the quintic
  Newton-Schulz iteration with tall matrices transposed, the shape scale, the
  decoupled weight decay, NorMuon, Muon+ row_col, and both cautious forms.
* ``adamw`` -- decoupled-weight-decay Adam with bias correction, the cautious
  wrapper, and bf16 moments (widened for the update, written back through
  ``storage``'s stochastic rounding).
* ``gradnorm`` -- the global gradient norm, the clip factor and the skip flag.
* ``storage`` -- the storage formats: decoding bf16 bit patterns, rounding
  float64 results to float32 / bf16 with round-to-nearest-even, and stochastic
  rounding to bf16 with a SplitMix64 counter hash.

Parity status: every function here is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle_pins.py`` (closed forms, the SVD reduction of
Newton-Schulz, invariants, brute force on tiny inputs) except where a docstring
says "parity unpinned".
"""
from . import storage, muon, adamw, gradnorm  # noqa: F401
