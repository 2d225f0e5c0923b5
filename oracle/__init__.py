"""Float64 CPU oracle (test infrastructure only; see muon_oracle's header)."""
from .muon_oracle import (OracleConfig, ns_poly, newton_schulz,  # noqa: F401
                          aurora_orthogonalize, power_sigma, momentum_nesterov, muon_update,
                          ns5_classic, classic_config, momentum_warmup)
