"""fp64 CPU oracle of the multi-token verify step (test infrastructure only)."""
