"""fp64 CPU GroupNorm oracle: test infrastructure only (see oracle.py)."""
