"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This package holds random draws and storage-format packing only -- none of
the attention, acceptance or quantization arithmetic.  Both the oracle side
and the GPU side receive the same arrays from here; neither side imports the
other.
"""
from .gen import *  # noqa: F401,F403
