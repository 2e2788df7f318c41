"""fp64 CPU oracle for the linear-memory relation-KL path (test infrastructure).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It shares no code with the HIP library and is never on
the product path.  See `relation_kl.py` for the definitions and citations.
"""
from .relation_kl import (  # noqa: F401
    relation_kl_head, relation_kl, relation_kl_xy, lse_rows, row_kl_rows, dx_rows,
    dx_rows_xy, dy_rows_xy, rope_rotate, rope_rotate_transpose, proj_bwd,
)
