"""MI355X-native NF4 double-quantized QLoRA linear (HIP for gfx950).

The compute path is the C-ABI library ``libqlora.so`` built from ``csrc/``;
:mod:`bit_nf4_quantized_double_amd.qlora` is a thin ctypes binding over it.
Importing this package does not load the library; the first call does, and
raises if it has not been built.
"""
