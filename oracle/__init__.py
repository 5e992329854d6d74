"""CPU oracle (test infrastructure only; see gpt2_oracle.py's header)."""
