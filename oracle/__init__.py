"""fp64 CPU oracle (test infrastructure only; never on the product path)."""
from .adam_oracle import ADAM_BETAS, ADAM_EPS, ADAM_LR, adam_scalars, adamw_step
from .muon_oracle import (NS_COEFFS, NS_EPS, NS_STEPS, aspect_factor, muon_step,
                          muon_update, nesterov_momentum, newton_schulz, ns_batched,
                          unview_blocks, view_blocks_of)

__all__ = ["ADAM_BETAS", "ADAM_EPS", "ADAM_LR", "NS_COEFFS", "NS_EPS", "NS_STEPS", "adam_scalars",
           "adamw_step", "aspect_factor", "muon_step", "muon_update", "nesterov_momentum",
           "newton_schulz", "ns_batched", "unview_blocks", "view_blocks_of"]
