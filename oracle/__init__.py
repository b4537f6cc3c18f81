"""CPU oracle of the activation-sparse gated FFN (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package; the product path never does.
"""
from .ffn import (ell_pack, ell_unpack, ffn_dense, ffn_dense_backward, ffn_sparse,
                  ffn_sparse_backward, gate_preact, l1_term, n_tiles,
                  relu, route, sparse_forward, twell_pack, twell_unpack, up_proj)

__all__ = ["ell_pack", "ell_unpack", "ffn_dense", "ffn_dense_backward", "ffn_sparse", "ffn_sparse_backward", "gate_preact", "l1_term", "n_tiles", "relu", "route",
           "sparse_forward", "twell_pack", "twell_unpack", "up_proj"]
