"""CPU oracle for mean-pooled Top-K block-routed sparse attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only the tests, the smoke check and the benchmark's CPU
baseline leg use it.  It shares no code with the HIP kernels or their Python
binding, and it imports neither.

Every function follows the pages it cites step by step, in plain NumPy
(float64 unless the pages fix fp32), with no blocking, fusion or reordering
beyond what the definitions state.  :mod:`oracle.sparse_attention` holds the
routed attention path (pooling, route scores, Top-K, exact and dense
attention, the video tail modes); :mod:`oracle.spark_summaries` holds the
Spark virtual summaries and the approximate branch for skipped blocks.  Each
module docstring lists what pins its functions.
"""

