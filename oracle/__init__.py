"""Float64 CPU oracle (test infrastructure only; see wkv7_oracle)."""
from .wkv7_oracle import (wkv7_step, wkv7_sequence, wkv7_forward,
                          wkv7_decode_batch, rel_max_err)

__all__ = ["wkv7_step", "wkv7_sequence", "wkv7_forward", "wkv7_decode_batch",
           "rel_max_err"]
