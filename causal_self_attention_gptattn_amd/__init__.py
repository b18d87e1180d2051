"""MI355X-native causal self-attention (placeholder; binding follows)."""
