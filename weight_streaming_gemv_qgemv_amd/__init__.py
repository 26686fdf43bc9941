"""MI355X (gfx950) dequant-on-use quantized GEMV and MoE block.

The compute lives in libcoli.so (hand-written HIP kernels behind a C ABI,
declared in include/coli.h).  `binding` is the thin ctypes layer over it;
`synth` draws the seeded synthetic inputs.  Importing this package loads
nothing: `binding` loads the library on first use and raises if it is
missing.
"""
__all__ = ["binding", "synth", "build"]
