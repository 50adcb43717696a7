"""CPU oracle (test infrastructure only; see spot_oracle)."""
