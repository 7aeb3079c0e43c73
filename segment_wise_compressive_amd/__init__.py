"""MI355X-native causal / decode / non-causal linear attention (phi = elu + 1)."""
