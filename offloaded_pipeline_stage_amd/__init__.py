"""MI355X (gfx950) implementation of one RoundPipe GPU-worker stage.

The hot path is the C-ABI library librp.so (include/rp.h) built from the HIP
sources in csrc/; ``binding`` is its ctypes binding and ``worker`` packs
weights and drives whole stages through it. Importing this package loads
nothing; the library is loaded on first use and its absence is an error.
"""

__all__ = ["binding", "worker", "build"]
