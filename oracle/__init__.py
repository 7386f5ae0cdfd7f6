"""Float64 CPU oracle for DropKV scoring (test infrastructure only)."""
