"""fixed_point_int8_amd: the fixed-point transformer forward pass of the
curta-core inference core ("The inference core" page) on MI355X (gfx950).

  binding  -- the C ABI of libfpi8 (include/fpi8.h), same names, marshalling only
  device   -- an artifact and a batch of run states in GPU memory (PyTorch plumbing)
  build    -- compiles libfpi8.so with hipcc for gfx950
"""
from . import binding  # noqa: F401
