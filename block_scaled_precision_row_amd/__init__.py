"""Block-scaled quantized linear layer (fp8r / nvfp4) for MI355X (gfx950).

The compute path lives in ``libbsq.so`` (hand-written HIP kernels behind a C
ABI declared in ``include/bsq.h``); ``_lib`` is a thin ctypes binding with the
same names. Importing the binding fails loudly if the library is missing.
"""
