"""MI355X-native DFlash block draft-and-verify step.

The compute lives in the HIP library ``libdflash.so`` (built from ``csrc/``); this
package holds its ctypes binding (``binding``), the workload shapes (``configs``)
and the seeded synthetic inputs (``synth``).
"""
__all__ = ["configs", "synth", "binding"]
