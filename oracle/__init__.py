"""fp64 CPU oracle for the Gated DeltaNet token mixer.

Test infrastructure only: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the product path.
"""
from .backward import recurrent_grads
from .gdn_oracle import (chunk_factors, chunked, decode_step, output_norm_gate, recurrent, sequence_bounds,
                         short_conv, unrolled, verify)

__all__ = ["recurrent", "chunked", "chunk_factors", "unrolled", "decode_step", "verify", "output_norm_gate",
           "short_conv", "recurrent_grads", "sequence_bounds"]
