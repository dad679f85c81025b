"""MiTA attention forward pass on AMD Instinct MI355X (gfx950).

The compute runs in ``libmita.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/mita.h``); ``mita`` is its thin Python binding.
"""
