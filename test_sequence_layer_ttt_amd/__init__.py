"""TTT layer inner loop on AMD Instinct MI355X (gfx950).

The computation lives in libttt.so (hand-written HIP kernels behind a C ABI,
declared in include/ttt.h); `ttt` is its thin Python binding and `gen` draws
seeded synthetic inputs. Importing the package does not load the library.
"""

__all__ = ["gen", "ttt"]
