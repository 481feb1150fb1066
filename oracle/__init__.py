"""CPU oracle for MSA block-sparse attention (test infrastructure only).

Only tests, the smoke check and the benchmark's CPU-baseline leg import this
package; the product library never does.
"""
from .msa_oracle import (block_scores, kept_keys, msa_forward, num_blocks,  # noqa: F401
                         query_positions, select_blocks, sparse_attention)
