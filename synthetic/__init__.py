"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle.

This package draws random numbers and lays out mask *parameters* (document
lengths, prefix lengths, answer cuts, block bitmaps).  It holds none of the
attention arithmetic and none of the mask semantics: the oracle turns a mask
spec into a predicate on its own, and the library turns it into a descriptor
on its own.
"""
from .inputs import *  # noqa: F401,F403
