"""ORACLE — test infrastructure only.

Plain CPU fp64 references for the ParaRNN/DEER hot path.  Only ``tests/``,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import this package; the product path (``nonlinear_rnn_amd``) never does,
and this package imports nothing from it.

* ``oracle.sequential`` — the definition: step-by-step application of the
  cell in double precision (C library ``liboracle.so``), and back-propagation
  through time for the gradients.
* ``oracle.deer`` — the DEER Newton solve written out in the order the pages
  derive it (residual, block-bidiagonal Jacobian, forward substitution, or a
  pairwise tree scan of affine maps), in numpy float64, for invariant and
  per-iteration checks.
* ``oracle.projection`` — the input projection u = W x + b per batch row in
  float64.

Parity status: every function here is pinned by tests in
``tests/test_oracle_pins.py`` against library routines (torch.nn.GRUCell /
LSTMCell with diagonal recurrent weights, scipy.signal.lfilter), closed
forms, finite differences and brute force; none is "parity unpinned".
"""
