"""MI355X-native DSA sparse-attention path (see binding module)."""
