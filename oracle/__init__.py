"""CPU oracle for the lightning-indexer hot path (test infrastructure only)."""
