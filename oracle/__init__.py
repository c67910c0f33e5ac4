"""Float64 CPU oracle for the diagonal linear RNN / diagonal SSM forward map.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code,
tables, constants or helpers with the HIP library; the two meet only through
the seeded input generators, which hold none of the method's arithmetic.

Every function here is a plain, slow, obviously correct restatement of what the
pages define, in float64, from the float32 input values promoted exactly:

* ``dlr``  -- the diagonal linear RNN (DLR) of "Simplifying and Understanding
  State Space Models with Diagonal Linear RNNs", section 2: the parameterisation
  of Lambda, the kernel K_j = sum_n w_n lambda_n^j, the real cast (and the
  DLR-prod cast Re K Im K of section 2.1), the causal convolution and the
  bidirectional sum; computed twice, as an O(L^2) direct sum
  and as a sequential recurrence; and the recurrence continued from a given
  state (streaming / one-token decode), returning the state it ends in.
* ``dlr_grad`` -- the gradients of that layer map at an output cotangent
  (du, d log_re, d log_im, dW, dD), from the chain rule on the same
  definitions.
* ``s5``   -- the multi-input multi-output diagonal SSM of "Simplified State
  Space Layers for Sequence Modeling", section 3, computed as a sequential
  recurrence and as a direct causal sum over a prefix; and its continuous-time
  form with a step size that changes from step to step (zero-order hold).

Parity status: every function is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle_pins.py`` (closed forms, a library DFT, brute-force
Toeplitz/circulant matrices and invariants).  No function is "parity unpinned".
"""

from .dlr import (  # noqa: F401
    dlr_lambda,
    dlr_kernel,
    dlr_kernel_cast,
    dlr_direct,
    dlr_recurrence,
    dlr_recurrence_state,
)
from .dlr_grad import dlr_backward  # noqa: F401
from .s5 import s5_recurrence, s5_direct_prefix, s5_recurrence_tv  # noqa: F401
