"""MI355X-native fused EM for Gaussian mixture models (placeholder until the binding lands)."""
