"""CPU oracle (test infrastructure only; never on the product path).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may import this package.  It is independent of the HIP library.
"""
from .sas_oracle import (  # noqa: F401
    BLOCK, pool_scores, select, select_row, mask_documents, bias_matrix, fwd_dense, fwd_gather,
    fwd_gather_block, gate_jacobian, bwd_dense, bwd_gather, bwd_gather_block,
    bwd_kv_block, reverse_lists, sas_forward_backward, decode, selected_pairs,
    blocks_of_documents, packed_geometry,
)
