"""libsala: the SALA hybrid attention hot path (linear + block-sparse layers) for MI355X.

Modules: ``sala`` (ctypes binding of libsala.so: the HIP kernels), ``inputs`` (seeded synthetic
workloads), ``build`` (hipcc build of libsala.so for gfx950).
"""
