"""CPU oracle for the AWQ scale search: test infrastructure only (see oracle.py)."""
