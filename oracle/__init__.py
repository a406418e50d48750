"""CPU oracle of the CSA indexer (test infrastructure only; see idx_oracle.c)."""
