"""Plain CPU oracle of the LSA indexer path (test infrastructure only)."""
