"""Local Mixture-of-Experts FFN forward on AMD Instinct MI355X (gfx950).

The compute path is the C-ABI library ``libmoe_ffn.so`` (hand-written HIP
kernels); ``moe`` holds its thin Python binding. ``inputs`` holds the seeded
synthetic-input generator. Importing the package loads nothing native; the
library is loaded on first use of ``moe``.
"""
