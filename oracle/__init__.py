"""fp64 CPU oracle for Soft-DTW: test infrastructure only (see oracle.py)."""
