"""MI355X-native pyramid Top-K block selection (PISA selection stage).

The compute path is the HIP library ``libpisa.so`` built from ``csrc/`` for
gfx950; ``ops`` is a thin ctypes binding over its C ABI (``include/pisa.h``).
``synth`` draws the seeded synthetic inputs.
"""
__all__ = ["ops", "synth"]
