"""nonlinear_rnn_amd — ParaRNN/DEER parallel-in-time Newton solve on MI355X.

The compute lives in ``libpararnn.so`` (hand-written HIP kernels for gfx950
behind a C ABI, declared in ``include/pararnn.h``); ``nonlinear_rnn_amd.pararnn``
is its thin Python binding.  ``nonlinear_rnn_amd.inputs`` draws the seeded
synthetic workloads.  Importing the package loads nothing; the binding loads
the library on first use and raises if it is missing.
"""
__all__ = ["pararnn", "inputs"]
