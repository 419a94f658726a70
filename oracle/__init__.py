"""CPU oracle for the CSA / HCA attention layer: fp64 NumPy, slow and plain.

This package is test infrastructure.  Only the test-suite, the smoke check and
the benchmark's CPU-baseline leg may import it; the library and its Python
binding never do, and it shares no code with them.

  formats  -- FP8 E4M3FN / BF16 / MXFP4 decode and encode
  csa      -- pooling, RMSNorm, RoPE, indexer, top-k, attention (vectorised)
  brute    -- scalar loop restatement for tiny inputs
  pipeline -- whole decode / prefill steps over generator inputs
"""
from . import formats, csa, brute, pipeline  # noqa: F401
