"""Double-precision CPU oracle for the gated delta rule.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
CPU-baseline leg of bench.py, never by the HIP package.
"""
from .oracle import (CHUNK, bwd, chunk_cumsum, chunk_form, fwd, fwd_split, last_threads,
                     num_chunks, token_recurrence_np)

__all__ = ["CHUNK", "bwd", "chunk_cumsum", "chunk_form", "fwd", "fwd_split", "last_threads",
           "num_chunks", "token_recurrence_np"]
