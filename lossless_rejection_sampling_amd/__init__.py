"""DSpark draft/verify round on AMD MI355X: hand-written HIP kernels for gfx950
behind a C ABI (include/dspark.h), with a thin ctypes binding.

Modules: ``dspark`` (binding), ``round`` (buffers and call order),
``workloads`` (seeded synthetic inputs), ``build`` (hipcc build)."""
