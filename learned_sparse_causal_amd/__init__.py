"""MI355X-native routed sparse causal attention (placeholder; binding below)."""
