"""CPU oracle for quantized-KV streaming decode attention (test infrastructure only)."""
