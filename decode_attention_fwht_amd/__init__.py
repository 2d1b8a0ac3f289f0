"""MI355X-native OmniKVQuant hot path: 2-bit KV-cache codec + fused decode attention."""
