"""CPU oracle for the Muon step — test infrastructure only (see muon_oracle.py).

Only the tests, the package's smoke check and the benchmark's CPU-baseline leg import
this package.  Every arithmetic function here is pinned by tests/test_oracle_*.py.  One
choice is a reading that no pin can fix and that does not affect parity:
canonical_orientation (which side of a non-square matrix is transposed so that the Gram
matrix is formed on the short side); only its consequences are pinned (the output is
transposed back, NS(X^T) = NS(X)^T).
"""
from .muon_oracle import *  # noqa: F401,F403
from .muon_oracle import __all__  # noqa: F401
