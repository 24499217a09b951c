"""MI355X-native gated delta-rule / diagonal Kalman Delta Network recurrence.

The compute path is the HIP library ``libkdn.so`` (C ABI declared in
``include/kdn.h``), reached through the ctypes binding in :mod:`.kdn`.
Importing this package loads nothing; the binding loads the library on first
use and raises if it is missing.
"""
__all__ = ["kdn", "synth"]
