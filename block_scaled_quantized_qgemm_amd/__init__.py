"""MI355X-native quantized linear layer (int8 per-token/per-channel and MXFP8)."""
