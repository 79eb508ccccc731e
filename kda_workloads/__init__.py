"""Synthetic KDA workloads: sizes as data (configs) and seeded input generators (gen).

Shared by the tests, the benchmark and the oracle-side checks; holds none of
the layer's arithmetic.
"""

from . import configs, gen  # noqa: F401
