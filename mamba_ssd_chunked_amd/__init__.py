"""MI355X-native Mamba-2 SSD chunked forward (float and persistent-INT8 paths)."""
