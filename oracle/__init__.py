"""CPU oracle (test infrastructure only; see pkv_oracle's header)."""
