"""CPU oracle (test infrastructure only; never imported by the product path)."""

from .oracle import backward, forward, fwd_bwd, rows_dh, rows_forward

__all__ = ["forward", "backward", "fwd_bwd", "rows_forward", "rows_dh"]
