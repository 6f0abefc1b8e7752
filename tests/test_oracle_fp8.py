"""Pins for the oracle's E4M3 decoder (CPU only).

The decoder (oracle/fp8.py) is written from the OCP 8-bit floating point
specification's field layout. These checks tie it to facts the
specification states about the format rather than to its own formula:
named extreme values, the NaN patterns, the absence of infinities, sign
symmetry, ordering, the spacing inside each binade, and the set of values
built another way (integer multiples of powers of two). A few plausible
mistakes (the other 8-bit E4M3 variant's bias, an off-by-one subnormal
scale, an exponent field read as all-ones-is-NaN) are planted in copies
below and must each fail one of these checks.
"""

import math

import numpy as np
import pytest
import torch

from oracle.fp8 import E4M3_NAN_CODES, E4M3_VALUES, e4m3_decode, e4m3_value


def check_named_values(table):
    """Values the specification names for E4M3."""
    return (table[0x00] == 0.0 and not math.copysign(1.0, table[0x00]) < 0
            and table[0x80] == 0.0 and math.copysign(1.0, table[0x80]) < 0
            and table[0x38] == 1.0            # E = 7, M = 0
            and table[0x40] == 2.0 and table[0xC0] == -2.0
            and table[0x7E] == 448.0          # largest finite
            and table[0xFE] == -448.0
            and table[0x08] == 2.0 ** -6      # smallest normal
            and table[0x07] == 7.0 / 8.0 * 2.0 ** -6   # largest subnormal
            and table[0x01] == 2.0 ** -9)     # smallest nonzero


def check_nan_and_inf(table):
    nan_codes = tuple(int(c) for c in np.flatnonzero(np.isnan(table)))
    return nan_codes == (0x7F, 0xFF) and not np.isinf(table).any()


def check_sign_and_order(table):
    pos = table[:0x7F]                        # codes 0x00 .. 0x7E
    neg = table[0x80:0xFF]
    return bool(np.all(np.diff(pos) > 0) and np.array_equal(neg, -pos))


def check_binade_spacing(table):
    # inside exponent field E >= 1 the 8 mantissas step by 2^(E - 10); the
    # subnormals step by 2^-9, continuing into the first binade
    for e in range(1, 16):
        codes = [(e << 3) | m for m in range(8) if not (e == 15 and m == 7)]
        vals = table[codes]
        if not np.all(np.diff(vals) == 2.0 ** (e - 10)):
            return False
    sub = table[0:9]
    return bool(np.all(np.diff(sub) == 2.0 ** -9))


def check_value_set(table):
    # positive finite E4M3 values: m * 2^-9 (m = 0..7) and (8 + m) * 2^(E - 10)
    # for E = 1..15, except the NaN pattern E = 15, m = 7
    want = {m * 2.0 ** -9 for m in range(8)}
    want |= {(8 + m) * 2.0 ** (e - 10) for e in range(1, 16) for m in range(8) if not (e == 15 and m == 7)}
    got = set(float(x) for x in table[:0x80] if not math.isnan(x))
    return got == want and len(got) == 127


CHECKS = [check_named_values, check_nan_and_inf, check_sign_and_order, check_binade_spacing, check_value_set]


@pytest.mark.parametrize("check", CHECKS, ids=lambda f: f.__name__)
def test_e4m3_decoder(check):
    assert check(E4M3_VALUES)


def test_e4m3_counts():
    finite = E4M3_VALUES[~np.isnan(E4M3_VALUES)]
    assert finite.size == 254
    assert np.unique(finite).size == 253           # +0 and -0 compare equal
    assert set(E4M3_NAN_CODES) == {0x7F, 0xFF}


def test_e4m3_values_are_exact_in_fp16_and_bf16():
    # the GPU path converts codes to the query's 16-bit type before its
    # products; that is exact only because every E4M3 value is an fp16 and a
    # bf16 value (3 mantissa bits, exponents 2^-9 .. 2^8)
    finite = E4M3_VALUES[~np.isnan(E4M3_VALUES)]
    assert np.array_equal(finite.astype(np.float16).astype(np.float64), finite)
    as_bf16 = torch.from_numpy(finite).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(as_bf16, finite)


def test_e4m3_decode_scale_and_types():
    codes = np.array([0x38, 0xC0, 0x01, 0x7E], dtype=np.uint8)
    assert np.array_equal(e4m3_decode(codes), [1.0, -2.0, 2.0 ** -9, 448.0])
    assert np.array_equal(e4m3_decode(torch.from_numpy(codes), scale=0.25), [0.25, -0.5, 2.0 ** -11, 112.0])
    with pytest.raises(TypeError):
        e4m3_decode(codes.astype(np.int32))
    with pytest.raises(ValueError):
        e4m3_value(256)


# ----------------------------------------------------------------- mutants

def _mutant_table(bias=7, sub_exp=None, nan_all_e15=False):
    def value(code):
        s = -1.0 if code & 0x80 else 1.0
        e, m = (code >> 3) & 0xF, code & 0x7
        if (e == 0xF and (nan_all_e15 or m == 0x7)):
            return math.nan
        if e == 0:
            return s * math.ldexp(m / 8.0, (1 - bias) if sub_exp is None else sub_exp)
        return s * math.ldexp(1.0 + m / 8.0, e - bias)
    return np.array([value(c) for c in range(256)], dtype=np.float64)


@pytest.mark.parametrize("mutant", [
    dict(bias=8),                 # the other E4M3 variant's exponent bias
    dict(sub_exp=-7),             # subnormals one binade too low
    dict(nan_all_e15=True),       # the whole top exponent taken as NaN
], ids=["bias8", "subnormal_scale", "e15_all_nan"])
def test_e4m3_mutants_are_caught(mutant):
    table = _mutant_table(**mutant)
    assert not all(check(table) for check in CHECKS)
