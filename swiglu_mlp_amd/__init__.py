"""MI355X-native ConvRot INT8 linear + fused SwiGLU MLP (binding filled in below)."""
