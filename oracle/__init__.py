"""CPU oracle of the SparsePR call (test infrastructure; see sparsepr_oracle)."""
