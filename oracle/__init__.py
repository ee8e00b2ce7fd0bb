"""fp64 CPU oracle of the gated-prefill path (test infrastructure only)."""
