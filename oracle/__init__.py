"""CPU float64 oracle for MLA decode (test infrastructure; see mla_oracle)."""
