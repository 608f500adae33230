"""CPU oracle of the Muon / SignMuon step -- test infrastructure only.

Imported by ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg
of ``bench.py``; never by the product package.
"""
from .muon_oracle import *  # noqa: F401,F403
from .muon_oracle import __all__  # noqa: F401
