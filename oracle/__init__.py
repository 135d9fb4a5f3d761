"""CPU oracle for the SparseSAM encoder-block hot path.

TEST INFRASTRUCTURE ONLY. Nothing in the product package may import, call or
execute anything under this directory; only the tests, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` use it. The
oracle imports nothing from the product either: the two share no code, only
the seeded inputs from ``synth``.
"""
from .sparsesam_oracle import *  # noqa: F401,F403
from .sparsesam_oracle import __all__  # noqa: F401
