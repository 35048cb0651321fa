"""MI355X-native retention operator (chunkwise forward, decode step, gated forward)."""
