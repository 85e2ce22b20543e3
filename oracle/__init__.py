"""CPU oracle of the quantized delta-rule decode step (test infrastructure only)."""
