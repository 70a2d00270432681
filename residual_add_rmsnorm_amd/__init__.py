"""libfusednorm for MI355X (gfx950): the fused tensor-parallel epilogue and the
segment RMSNorms as hand-written HIP kernels behind a C ABI.

Modules:
  fusednorm   the Python binding of the C ABI (include/fusednorm.h); importing
              it loads libfusednorm.so and fails if the library is not built
  workloads   seeded synthetic inputs of the benchmark and test workloads
  _build      builds libfusednorm.so in-tree with hipcc

Nothing is imported here, so the package can be imported without a GPU.
"""
