"""fp64 CPU oracle for KDA (test infrastructure only; see oracle.py)."""
