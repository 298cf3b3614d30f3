"""CPU oracle of the MoE layer forward (test infrastructure only; see moe_oracle)."""
