"""CPU oracle for the Polar Attention forward (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg import this
package; the GPU library does not, and the two share no code.
"""
from .polar_oracle import *  # noqa: F401,F403
from .polar_oracle import __all__  # noqa: F401
from .polar_backward import polar_attention_backward, row_coefficients  # noqa: F401,E402

from .polar_variants import (DEFAULT_VARIANT, merge_variant, polar_attention_variant,  # noqa: F401,E402
                             split_statistics_variant, variant_of)

__all__ = list(__all__) + ["polar_attention_backward", "row_coefficients", "DEFAULT_VARIANT", "merge_variant",
                           "polar_attention_variant", "split_statistics_variant", "variant_of"]
