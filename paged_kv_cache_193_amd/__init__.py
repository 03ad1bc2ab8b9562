"""MI355X-native paged KV-cache attention (placeholder until the HIP library lands)."""
