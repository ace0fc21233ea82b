"""CPU oracle (test infrastructure only; never imported by the product path)."""

from .mlp import mlp_backward, mlp_cols_grads, mlp_fwd_bwd, mlp_forward, mlp_rows_dx, mlp_rows_forward
from .oracle import backward, cols_dW, forward, fwd_bwd, rows_dh, rows_forward

__all__ = ["forward", "backward", "fwd_bwd", "rows_forward", "rows_dh", "cols_dW",
           "mlp_forward", "mlp_backward", "mlp_fwd_bwd", "mlp_rows_forward", "mlp_rows_dx", "mlp_cols_grads"]
