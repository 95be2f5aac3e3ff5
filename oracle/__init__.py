"""CPU oracle for the causal Based forward. Test infrastructure only: see based_oracle.py."""
from .based_oracle import (  # noqa: F401
    DEN_GUARD, MAX_ABS_TOL, REL_L2_TOL, bf16_to_f64, resolve_scale, taylor_weight, phi,
    based_ref_direct, based_ref_direct_rows, based_ref_chunked, based_ref_chunked_state, based_ref_decode_step,
    based_ref_rational, rational_to_f64, feature_dim,
    errors, passes_gate,
)
