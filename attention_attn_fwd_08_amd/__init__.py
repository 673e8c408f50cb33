"""MI355X-native fused attention forward (placeholder until the binding lands)."""
