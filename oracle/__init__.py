"""CPU oracle (test infrastructure only; see dsa_oracle)."""
