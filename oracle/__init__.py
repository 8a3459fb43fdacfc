"""CPU oracle for the MoE layer (test infrastructure only; see moe_oracle)."""
