"""CPU oracle for the CSA / HCA compressed-attention path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links this
package: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code with the HIP library; both are fed from the
seeded generators in ``synthgen``.

Parity status: every function here is pinned by a CPU test against values printed on
the pages or against closed forms and brute force (see ``tests/test_oracle_pins.py``).
"""
from . import kvcache  # noqa: F401
from .csahca import (  # noqa: F401
    E2M1_TABLE,
    E4M3FN_TABLE,
    attend,
    csa_rows,
    decode,
    decode_bf16,
    decode_e4m3fn,
    decode_mxfp4,
    entry_counts,
    entry_positions,
    grouped_out_proj,
    hca_rows,
    index_scores,
    norm_rope,
    pool,
    pool_overlap,
    rmsnorm,
    rope_tail,
    topk,
    visible,
    window_positions,
)
