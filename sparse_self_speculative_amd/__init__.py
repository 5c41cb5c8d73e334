"""SparseSpec attention hot path for AMD MI355X (gfx950).

The product is libsspec.so (HIP kernels behind the C ABI of include/sspec.h)
and its thin binding, `sparse_self_speculative_amd.sspec`.  Build the
library with `python -m sparse_self_speculative_amd.build`.
"""
