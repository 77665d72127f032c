"""CPU oracle for mean-pooled Top-K block-routed sparse attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only the tests, the smoke check and the benchmark's CPU
baseline leg use it.  It shares no code with the HIP kernels or their Python
binding, and it imports neither.

Every function follows the pages it cites step by step, in plain NumPy
(float64 unless the pages fix fp32), with no blocking, fusion or reordering
beyond what the definitions state.  Parity status of each function is listed
in the module docstring of :mod:`oracle.sparse_attention`.
"""

