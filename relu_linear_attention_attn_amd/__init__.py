"""ReLU linear self-attention forward (Sana Linear DiT) for AMD MI355X.

The compute runs in hand-written HIP kernels behind a C ABI
(``libsana_linattn.so``, declared in ``include/sana_linattn.h``); this package
is a thin ctypes binding plus the seeded workload generator.
"""
