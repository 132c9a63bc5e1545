"""CPU oracle (test infrastructure only; see kvx_oracle)."""
