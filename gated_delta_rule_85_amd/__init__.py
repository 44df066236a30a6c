"""MI355X (gfx950) gated delta rule chunked prefill.

The operator (FlashQLA's GDN chunked prefill) runs in libgdr.so, hand-written
HIP kernels behind the C ABI of include/gdr.h; this package is a thin
PyTorch-facing binding of it.
"""
from .api import (SavedForBackward, chunk_bound, chunk_gated_delta_rule, chunk_gated_delta_rule_bwd,
                  chunk_gated_delta_rule_fwd, num_chunks)

__all__ = ["chunk_gated_delta_rule", "chunk_gated_delta_rule_fwd", "chunk_gated_delta_rule_bwd",
           "num_chunks", "chunk_bound", "SavedForBackward"]
