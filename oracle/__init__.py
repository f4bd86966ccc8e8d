"""CPU oracle (test infrastructure only; see ds_oracle.py)."""
