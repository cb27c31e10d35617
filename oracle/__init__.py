"""CPU oracle (test infrastructure only; see zr_oracle.py)."""
