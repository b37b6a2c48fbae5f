"""CPU oracle (test infrastructure only; see cq_oracle.py)."""
