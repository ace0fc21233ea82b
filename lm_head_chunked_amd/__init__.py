"""MI355X-native fused LM-head + cross-entropy (chunked NLL) loss."""
