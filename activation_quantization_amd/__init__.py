"""MI355X-native online KV-cache / activation quantizer (nsep+pchan, randomized Hadamard).

The compute path is the C-ABI library libkvq.so (hand-written HIP kernels for gfx950);
this package holds its thin ctypes binding and the seeded synthetic input generator.
"""
