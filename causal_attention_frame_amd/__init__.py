"""MI355X-native frame-block-causal attention with a reference-anchored KV ring."""
