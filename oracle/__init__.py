"""CPU oracle for RMSNorm forward and backward -- TEST INFRASTRUCTURE ONLY.

This package is the yardstick the HIP library is checked against. It is not
part of the product path: only the test suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import it.
It shares no code with the HIP library (``backward_rmsnorm_fwd_amd``) and
imports nothing from it; the library never imports this package.

Contents (the three roles follow the torchtitan "kernel-numerics-verifier"
page, section "核心方法" (core method): golden / reference / target):

* ``golden``    -- the definition of RMSNorm forward and backward written out
                   in float64 with NumPy, fed the very same low-precision
                   inputs promoted losslessly to float64.
* ``reference`` -- an eager PyTorch-CPU implementation in the kernel's dtype
                   with float32 intermediates; it measures how close a correct
                   same-precision implementation gets to the golden.
* ``layernorm`` -- the same two roles (float64 golden, float32 same-dtype
                   reference) for LayerNorm, the sibling operation.
* ``fused``     -- the neighbours fused with RMSNorm: the residual add before
                   it and the cast of its output to a narrower dtype after
                   it, composed from the pinned RMSNorm golden and reference
                   with PyTorch's own add and cast.
* ``gate``      -- the correctness gate of that page (section "正确性判据",
                   the correctness criterion) with its conditioning check,
                   plus the constants it uses, fixed before any kernel ran.

Parity status: every public function of ``golden``, ``layernorm`` and
``fused`` is pinned (``tests/test_layernorm_oracle.py``,
``tests/test_fused_oracle.py`` and ``tests/test_cast_oracle.py`` for the
latter two) by the
``-m "not gpu"`` tests in ``tests/test_oracle_pins.py`` (printed worked
examples, closed forms, invariants, central differences, and PyTorch's own
``rms_norm`` with autograd in float64).  ``reference`` is pinned against the
golden and against autograd of itself.  No function here is "parity unpinned".
"""
