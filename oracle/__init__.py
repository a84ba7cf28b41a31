"""CPU oracle of the MoE expert stage (test infrastructure only)."""
