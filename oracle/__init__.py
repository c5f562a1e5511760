"""fp64 CPU oracle for HiKVP attention (test infrastructure only)."""
