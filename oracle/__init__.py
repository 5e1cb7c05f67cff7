"""CPU oracle for MLA decode -- test infrastructure only (see mla_oracle)."""
