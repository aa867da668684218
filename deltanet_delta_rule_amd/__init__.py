"""MI355X-native DeltaNet delta-rule operator (HIP/gfx950)."""
