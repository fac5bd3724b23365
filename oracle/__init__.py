"""CPU oracle (test infrastructure only): see gla_oracle.py, swiglu_oracle.py and saga_oracle.py."""

from .gla_oracle import (  # noqa: F401
    SCAN_B2T,
    SCAN_L2R,
    SCAN_R2L,
    SCAN_ROTATE_BATCH,
    SCAN_T2B,
    batch_directions,
    gla_backward,
    gla_forward,
    log_alpha_from_logits,
    scan_order,
)
from .swiglu_oracle import depthwise_conv3x3, silu, spatial_swiglu  # noqa: F401
from .saga_oracle import saga_forward, saga_kv  # noqa: F401
