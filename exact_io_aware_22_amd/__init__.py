"""MI355X-native exact tiled attention forward and split-KV decode.

The device work runs in hand-written HIP kernels for gfx950 inside `libfa.so`
(C ABI declared in include/fa.h). This package holds the thin ctypes binding
(`exact_io_aware_22_amd.fa`), the library build step (`build`) and the seeded
workload generator (`workloads`). Importing the package loads nothing; the
library is loaded on the first binding call and a missing library is an error.
"""
