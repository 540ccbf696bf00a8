"""bfloat16 bit patterns -> exact float64 values.  Oracle / test infrastructure.

A bfloat16 value is the upper half of an IEEE-754 binary32 value: sign, the
8-bit exponent and the top 7 mantissa bits.  Widening is therefore exact:
put the 16 bits in the high half of a 32-bit word, read it as binary32, and
widen binary32 to binary64 (also exact).  The pages store K/V and Q in bf16
(InferX, "Measured" and "The kernels underneath": bf16 serving; llm-infer,
"Serving Details": --dtype bfloat16).
"""

import numpy as np


def to_f64(bits):
    """uint16 (or int16) array of bf16 bit patterns -> float64 array, exact."""
    b = np.asarray(bits)
    if b.dtype == np.int16:
        b = b.view(np.uint16)
    if b.dtype != np.uint16:
        raise TypeError("bf16 bit patterns must be uint16 or int16, got %s" % b.dtype)
    words = b.astype(np.uint32) << np.uint32(16)
    # signalling-NaN patterns widen to NaN; numpy would warn about the cast
    with np.errstate(invalid="ignore"):
        return words.view(np.float32).astype(np.float64)
