"""gradient_compression_dnn_amd — binding placeholder (filled in with the C-ABI)."""
