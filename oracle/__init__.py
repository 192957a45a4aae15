"""Float64 CPU oracle for FLCE (test infrastructure only; never on the product path)."""
from .flce_oracle import (  # noqa: F401
    ce_ref,
    ce_rows_ref,
    check_targets,
    flce_brute_force,
    flce_ref,
    flce_ref_rowblocks,
    flce_rows_ref,
    row_lse,
)
from .orpo_oracle import orpo_loss_only, orpo_ref, orpo_terms  # noqa: F401,E402
