"""One MI355X rank of a folded tensor+sequence parallel (TSP) transformer layer.

The compute lives in libtsp.so (HIP for gfx950, C ABI in include/tsp.h);
`tsp` is its ctypes binding and `build` compiles it.
"""
from . import tsp  # noqa: F401
