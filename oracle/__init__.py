"""CPU fp64 oracle for the LRM-pruned MoE expert backward (test infrastructure only)."""
