"""MI355X-native Mamba2 SSD selective-state-space scan (binding package)."""
