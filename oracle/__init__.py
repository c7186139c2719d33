"""fp64 CPU oracle (test infrastructure only; see e2ttt_oracle's header)."""
from .e2ttt_oracle import (KINDS, LOSSES, brute_force, chunk_coefficients, chunk_coefficients_nomomentum,
                           chunk_forward, chunk_mean, closed_form_transition, fast_weight_forward, grad_factors,
                           pack, param_count, rel_err, token_grads, unpack, weighted_grad_sum)
from .e2ttt_backward import chunk_backward

__all__ = ["KINDS", "LOSSES", "brute_force", "chunk_coefficients", "chunk_coefficients_nomomentum",
           "chunk_backward", "chunk_forward", "chunk_mean", "closed_form_transition", "fast_weight_forward", "grad_factors",
           "pack", "param_count", "rel_err", "token_grads", "unpack", "weighted_grad_sum"]
