"""MI355X-native MXFP8 / MXFP6 linear layer (placeholder; binding added below)."""
