"""CPU oracle for the HSA iteration: test infrastructure only (see hsa_oracle)."""
