"""MI355X-native sparse-attention decode step (DeepSeek-V4 style)."""
