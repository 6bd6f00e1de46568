"""fp64 CPU oracle of the AXELRAM hot path (test infrastructure only)."""
