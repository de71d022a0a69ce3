"""SparsePR attention call for AMD Instinct MI355X (gfx950): HIP kernels behind a C ABI.

``_lib`` is the ctypes binding of libsparsepr.so (include/sparsepr.h); ``call.SparsePR``
wraps one configuration with torch-allocated buffers; ``synth`` draws seeded inputs;
``configs`` lists the workloads.
"""
