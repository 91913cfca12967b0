"""CPU oracle for the Muon step — test infrastructure only (see muon_oracle.py).

Only the tests, the package's smoke check and the benchmark's CPU-baseline leg import
this package.  Parity of every function here is pinned by tests/test_oracle_*.py; no
function is "parity unpinned".
"""
from .muon_oracle import *  # noqa: F401,F403
from .muon_oracle import __all__  # noqa: F401
