"""CPU oracle for the byte-split BF16 codec (test infrastructure only)."""
