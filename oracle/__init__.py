"""CPU fp64 oracle (test infrastructure only; see vsa_oracle)."""
