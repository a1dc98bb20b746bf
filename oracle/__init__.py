"""CPU oracle for MLA (test infrastructure only; see mla_oracle's header)."""
