"""CPU oracle for one DeepSeek-Sparse-Attention layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this package: only the tests, the smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code, constants or helpers with the HIP
library or its Python binding, and neither side imports the other.

Contents:
  dsa_oracle  -- pooled indexer keys, indexer scores, full-sort top-k, key-set
                 expansion, explicit-softmax sparse attention forward and
                 backward, all in float64.
  zigzag      -- causal work counts for contiguous and zig-zag sequence splits.

Every function is pinned by a test against something other than itself; the
list of pins and the one unpinned item are in the module docstrings.
"""
from . import dsa_oracle, zigzag  # noqa: F401
