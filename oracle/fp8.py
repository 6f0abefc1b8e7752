"""8-bit floating-point K/V codes (OCP E4M3), decoded to float64.

TEST INFRASTRUCTURE ONLY (see the package docstring): the decode attention
oracle takes float K/V, and this module turns stored codes into those
floats, so that a check of the fp8-KV decode path is the plain float64
decode of the decoded values.

Reading. "The Online Softmax Recurrence" (section "Where it breaks") says
the statistics stay fp32 when Q, K and V are FP8 or BF16, but the pages fix
no FP8 format or scaling. The reading taken here is the common KV-cache
layout: K and V stored as one byte per element in the OCP 8-bit floating
point format E4M3, each tensor with one fp32 scale (k_scale, v_scale); the
element with code c stands for e4m3(c) * scale.

E4M3, from the OCP 8-bit floating point specification: bit 7 is the sign,
bits 6-3 the exponent field E (bias 7), bits 2-0 the mantissa field M.
  E = 0:               (-1)^s * (M / 8) * 2^(1 - 7)       (subnormal, and zero)
  0 < E, not E=15,M=7: (-1)^s * (1 + M / 8) * 2^(E - 7)
  E = 15 and M = 7:    NaN (the only NaN pattern per sign; no infinities)
so the largest finite magnitude is (1 + 6/8) * 2^8 = 448 and the smallest
nonzero one 2^-9.
"""

import math

import numpy as np

E4M3_BIAS = 7
E4M3_NAN_CODES = (0x7F, 0xFF)


def e4m3_value(code):
    """The value of one E4M3 code (an int in 0..255) as a Python float."""
    code = int(code)
    if not 0 <= code <= 255:
        raise ValueError(f"E4M3 code out of range: {code}")
    negative = (code >> 7) & 1
    exponent_field = (code >> 3) & 0xF
    mantissa_field = code & 0x7
    if exponent_field == 0xF and mantissa_field == 0x7:
        return math.nan
    if exponent_field == 0:
        magnitude = math.ldexp(mantissa_field / 8.0, 1 - E4M3_BIAS)
    else:
        magnitude = math.ldexp(1.0 + mantissa_field / 8.0, exponent_field - E4M3_BIAS)
    return -magnitude if negative else magnitude


# Value of every code, index = code.
E4M3_VALUES = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_decode(codes, scale=1.0):
    """float64 values of an array of E4M3 codes (uint8, numpy or torch),
    multiplied by ``scale`` (the tensor's fp32 scale)."""
    if hasattr(codes, "detach"):
        codes = codes.detach().cpu().numpy()
    codes = np.asarray(codes)
    if codes.dtype != np.uint8:
        raise TypeError(f"E4M3 codes must be uint8, got {codes.dtype}")
    return E4M3_VALUES[codes] * float(scale)
