"""Decoding of the stored number formats into fp64, written from their definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages fix only that attention runs in BF16 and that the KV cache may be
FP8 (Kimi K3 on MI355X, section 4 table notes "BF16 attention"; section 2 and
"Benchmark configuration" use "FP8 KV").  The FP8 flavour is read as OCP
E4M3FN (bias 7, no infinities, S.1111.111 is NaN), the FP8 format that gfx950
decodes natively.  These decoders are the oracle's own and share nothing with
the HIP path.
"""

import numpy as np


def bf16_bits_to_f64(bits):
    """bfloat16 bit patterns (uint16) -> fp64 values.

    bfloat16 is the upper half of an IEEE-754 binary32: the value is the
    binary32 whose high 16 bits are ``bits`` and whose low 16 bits are zero.
    The conversion to fp64 is exact.
    """
    bits = np.asarray(bits, dtype=np.uint16)
    wide = bits.astype(np.uint32) << np.uint32(16)
    return wide.view(np.float32).astype(np.float64)


def e4m3fn_codes_to_f64(codes):
    """OCP FP8 E4M3FN codes (uint8) -> fp64 values.

    Layout S EEEE MMM, exponent bias 7.
      E == 0            : subnormal, (-1)^S * 2^-6 * M/8
      E in 1..15        : normal,    (-1)^S * 2^(E-7) * (1 + M/8)
      E == 15 and M == 7: NaN (the format has no infinities)
    """
    codes = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((codes >> 7) & 1, -1.0, 1.0)
    exp = (codes >> 3) & 0xF
    man = (codes & 0x7).astype(np.float64)
    normal = np.ldexp(1.0 + man / 8.0, (exp - 7).astype(np.int64))
    subnormal = np.ldexp(man / 8.0, -6)
    mag = np.where(exp == 0, subnormal, normal)
    mag = np.where((exp == 15) & (man == 7), np.nan, mag)
    return sign * mag
