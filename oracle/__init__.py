"""CPU oracle of the MoE layer forward pass (test infrastructure only; see moe_oracle.py)."""
