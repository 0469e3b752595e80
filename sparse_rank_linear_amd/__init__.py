"""MI355X-native SALR linear layer (the HIP library and its binding follow)."""
