"""CPU oracles (test infrastructure only; see wkv7_oracle and q8_oracle)."""
from .wkv7_oracle import (wkv7_step, wkv7_sequence, wkv7_forward,
                          wkv7_decode_batch, rel_max_err)
from .q8_oracle import roundf, quantize_rows, q8_matmul, q8_linear

__all__ = ["wkv7_step", "wkv7_sequence", "wkv7_forward", "wkv7_decode_batch",
           "rel_max_err", "roundf", "quantize_rows", "q8_matmul", "q8_linear"]
