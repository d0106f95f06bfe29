"""float64 CPU oracle of the Mamba-3 forward path and its adjoints.

Test infrastructure: only the tests, the smoke check and the benchmark's CPU
baseline import this package.  It shares no code with the HIP library.
"""

from .m3_oracle import (  # noqa: F401
    MIMO_NORM_EPS,
    PreprocessConfig,
    SsmConfig,
    mimo_scan,
    mimo_step,
    parity_error,
    preprocess,
    preprocess_width,
    rotate,
    sigmoid,
    silu,
    siso_scan,
    siso_step,
    softplus,
)
from .m3_backward import PREPROCESS_OUTPUTS, mimo_backward, preprocess_backward, siso_backward  # noqa: F401
