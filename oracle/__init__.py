"""CPU oracle (test infrastructure only; see demo_oracle's header)."""
