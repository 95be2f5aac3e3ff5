"""MI355X-native causal Based forward (2nd-order Taylor linear attention) on hand-written HIP kernels.

The compute path lives in libbased.so (include/based.h); this package is its thin Python binding.
"""
from .based import Timer, based_decode_step, based_forward, feature_dim, plan, workspace_bytes  # noqa: F401
