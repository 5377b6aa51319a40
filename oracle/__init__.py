"""fp64 CPU oracle for the selective state-space scan.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, sequential
reference that the GPU path is checked against.  Only the test-suite, the
smoke check and the CPU-baseline leg of the benchmark may import it; the
product path never does, and the two share no code.

The arithmetic lives in ``ssm_ref.c`` (plain C, fp64); ``ref.py`` marshals
numpy arrays into it.  Parity pins are in ``tests/test_oracle_pins.py``.
``bwd.py`` is the backward pass: fp64 automatic differentiation (torch, CPU)
of its own transcription of the forward, pinned in ``tests/test_oracle_bwd.py``
against the C oracle's forward and central finite differences of it.
``ssm_ref.c`` also holds a second backward, ``ssm_ref_scan_bwd`` (``ref.scan_bwd``):
the hand-derived adjoint recurrence in C, threaded over channels, fast enough
for whole layers; it is pinned in ``tests/test_oracle_bwd_c.py`` against
central finite differences of the C forward, the relay example by hand and
the automatic-differentiation backward, with planted mistakes in
``tests/test_oracle_mutants.py``.
``ssd.py`` is the Mamba-2 SSD layer in its quadratic masked-matrix form (numpy),
pinned in ``tests/test_oracle_ssd.py`` against the C oracle's recurrence.

Pin status.  The trapezoidal (Mamba-3) scan is partly pinned: its tests fix the
step as read (impulse response, constant-input closed form, second-order
convergence, the A = 0 cumulative trapezoid), but the pages leave its three
coefficients undefined, so that this reading is the paper's is not checkable.
Full-size outputs with random inputs have no printed value to compare with;
they rest on the pinned functions.
"""
