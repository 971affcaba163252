"""fp64 CPU oracle of the TriAttention prune step (test infrastructure only)."""
