"""MI355X (gfx950) exact attention forward: HIP kernels behind a C ABI.

``exact_attention_95_amd.fa`` is the ctypes binding of include/fa.h;
``exact_attention_95_amd.inputs`` draws the seeded synthetic workloads;
``exact_attention_95_amd.build`` compiles ``libfa.so`` with hipcc.
Importing this package loads nothing: the library is opened on first use.
"""
