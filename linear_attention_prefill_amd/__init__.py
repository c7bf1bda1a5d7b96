"""MI355X-native KDA (Kimi Delta Attention) chunked prefill and decode."""
