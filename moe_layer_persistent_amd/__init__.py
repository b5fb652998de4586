"""MI355X-native MoE decoder-layer verify step (package root)."""
