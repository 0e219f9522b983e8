"""MI355X-native EQ-Linear forward (placeholder; the binding is added with the HIP library)."""
