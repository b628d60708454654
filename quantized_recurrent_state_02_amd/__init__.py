"""Compressed recurrent-state decode for GDN / KDA on MI355X (gfx950).

The compute path is the HIP library ``libqrs.so`` (sources in ``csrc/``,
declarations in ``include/qrs.h``); ``binding`` is a thin ctypes layer over
its C ABI, and ``inputs`` holds the seeded synthetic workloads.  Importing the
package does not load the library; the first call into ``binding`` does, and
fails loudly if it has not been built.
"""

__all__ = ["binding", "inputs"]
