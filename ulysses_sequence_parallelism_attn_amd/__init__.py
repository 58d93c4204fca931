"""MI355X-native per-rank Ulysses attention: HIP kernels behind a C ABI.

The compute path lives in ``libulattn.so`` (built from ``csrc/`` with hipcc for
gfx950); :mod:`.binding` is a thin ctypes layer over its ``extern "C"`` entry
points.  Importing this package loads nothing; the library is opened on first
use and the binding raises if it has not been built.
"""

__all__ = ["binding", "synth"]
