"""SLA2 sparse-linear attention forward for AMD MI355X (gfx950).

The compute lives in libsla2.so (hand-written HIP kernels behind the C ABI in
include/sla2.h); `sla2` is its thin ctypes binding, `workloads` the seeded
synthetic inputs, `build` the in-tree hipcc build.
"""
