"""MI355X-native selective state-space scan (Mamba selective scan) on gfx950.

The compute path is the C-ABI library ``libssmscan.so`` built from
``csrc/``; ``ops`` is a thin ctypes binding with the same entry-point names.
Importing this package loads nothing; the library is opened on first use.
"""
__all__ = ["inputs", "ops"]
