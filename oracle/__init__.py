"""CPU oracle for the Polar Attention forward (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg import this
package; the GPU library does not, and the two share no code.
"""
from .polar_oracle import *  # noqa: F401,F403
from .polar_oracle import __all__  # noqa: F401
from .polar_backward import polar_attention_backward, row_coefficients  # noqa: F401,E402

__all__ = list(__all__) + ["polar_attention_backward", "row_coefficients"]
