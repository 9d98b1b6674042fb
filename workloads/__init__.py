"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and the benchmark.

This package builds the four boundary vectors (LTS, LTE, UTS, UTE) of each structured mask
family and the Q/K/V/dO tensors from fixed seeds.  It holds none of the attention arithmetic,
none of the tile classification and none of the localisation: those live in ``oracle/`` (the
CPU reference) and in the HIP library, which share no code.
"""

from . import masks, configs  # noqa: F401
