"""fp64 CPU oracle (test infrastructure only; never on the product path)."""
from .muon_oracle import (NS_COEFFS, NS_EPS, NS_STEPS, aspect_factor, muon_step,
                          muon_update, nesterov_momentum, newton_schulz, ns_batched,
                          unview_blocks, view_blocks_of)

__all__ = ["NS_COEFFS", "NS_EPS", "NS_STEPS", "aspect_factor", "muon_step", "muon_update",
           "nesterov_momentum", "newton_schulz", "ns_batched", "unview_blocks", "view_blocks_of"]
