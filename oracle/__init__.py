"""fp64 CPU oracle of the gated delta-rule layer (test infrastructure only)."""
from .gdn_oracle import (EPS, l2norm_rows, recurrent_fwd, recurrent_bwd,  # noqa: F401
                         chunk_fwd)
